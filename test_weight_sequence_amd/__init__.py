"""MI355X-native TTT-Linear / TTT-MLP inner-loop scan.

The compute path is the HIP library under csrc/ (built to libttt.so) behind a C ABI;
`ops` is its thin ctypes binding. Importing this package loads nothing.
"""
