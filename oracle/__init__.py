"""fp64 CPU oracle for the TTT inner-loop scan (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import this
package. It shares no code with the HIP path.
"""
from .ttt_oracle import (OracleConfig, f_apply, gelu, gelu_prime, inner_forward,  # noqa: F401
                         l2_normalize_units, lact_apply, lact_token_grad, layer_norm, scan,
                         scan_lact, scan_momentum, scan_outer_grads, silu, silu_prime,
                         token_loss_and_grad)
