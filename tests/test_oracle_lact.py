"""Pins of the oracle's large-chunk SwiGLU TTT layer (scan_lact: "Test-Time Training(TTT)과 LLM
메모리", section "LaCT", Eq. 6/7/4/8/2) against library routines, finite differences and closed
forms. The independent reference below is written in the page's column-vector notation with
torch.nn.functional.silu, torch.autograd and torch.nn.functional.normalize."""
import pytest
import torch
import torch.nn.functional as F

from oracle import l2_normalize_units, lact_apply, lact_token_grad, scan_lact, silu, silu_prime

DT = torch.float64


def _inputs(N, T, d, h, seed):
    g = torch.Generator().manual_seed(seed)
    Q, K, V = (torch.randn(N, T, d, generator=g, dtype=DT) / d ** 0.5 for _ in range(3))
    eta = 0.5 * torch.sigmoid(torch.randn(N, T, generator=g, dtype=DT))
    W = (torch.randn(N, d, h, generator=g, dtype=DT) / d ** 0.5,
         torch.randn(N, h, d, generator=g, dtype=DT) / h ** 0.5,
         torch.randn(N, d, h, generator=g, dtype=DT) / d ** 0.5)
    return Q, K, V, eta, W


def _lib_f(x, P1, P2, P3):
    """Page notation: f_W(x) = W2 [SiLU(W1 x) o (W3 x)], x a column vector [d], W1, W3 [h, d],
    W2 [d, h]."""
    return P2 @ (F.silu(P1 @ x) * (P3 @ x))


def _lib_scan(Q, K, V, eta, W, chunk, apply="after"):
    """One head at a time: autograd of the chunk's eta-weighted loss -f(k).v at the chunk-start
    weights, then W - g with every row (output unit) normalised by F.normalize."""
    N, T, d = Q.shape
    Zs, WTs = [], []
    for n in range(N):
        P = [W[0][n].T.clone(), W[1][n].T.clone(), W[2][n].T.clone()]
        out = []
        for i in range(T // chunk):
            Pl = [p.detach().clone().requires_grad_(True) for p in P]
            L = sum(eta[n, t] * (-_lib_f(K[n, t], *Pl) @ V[n, t]) for t in range(i * chunk, (i + 1) * chunk))
            g = torch.autograd.grad(L, Pl)
            Pn = [F.normalize(p - gp, dim=1) for p, gp in zip(P, g)]
            use = Pn if apply == "after" else P
            out += [_lib_f(Q[n, t], *use) for t in range(i * chunk, (i + 1) * chunk)]
            P = [p.detach() for p in Pn]
        Zs.append(torch.stack(out))
        WTs.append((P[0].T, P[1].T, P[2].T))
    return torch.stack(Zs), tuple(torch.stack([w[k] for w in WTs]) for k in range(3))


def rel(a, b):
    return ((a - b).norm() / b.norm()).item()


def test_silu_and_derivative():
    x = torch.linspace(-8, 8, 401, dtype=DT)
    assert rel(silu(x), F.silu(x)) <= 1e-15
    h = 1e-6
    fd = (F.silu(x + h) - F.silu(x - h)) / (2 * h)
    assert (silu_prime(x) - fd).abs().max().item() <= 1e-9


def test_token_gradient_matches_autograd():
    Q, K, V, eta, W = _inputs(3, 1, 8, 24, seed=1)
    g = lact_token_grad(K[:, 0], V[:, 0], W)
    for n in range(3):
        P = [W[0][n].T.clone().requires_grad_(True), W[1][n].T.clone().requires_grad_(True),
             W[2][n].T.clone().requires_grad_(True)]
        L = -_lib_f(K[n, 0], *P) @ V[n, 0]
        ga = torch.autograd.grad(L, P)
        for k in range(3):
            assert rel(g[k][n], ga[k].T) <= 1e-13, k


def test_chunk_gradient_matches_finite_differences():
    """The summed, eta-weighted chunk gradient (Eq. 4) against central differences of the
    chunk loss along random directions, on a tiny head."""
    Q, K, V, eta, W = _inputs(1, 6, 4, 8, seed=2)

    def loss(Wx):
        return sum((eta[0, t] * -(lact_apply(K[:, t], Wx)[0] @ V[0, t])) for t in range(6))

    g = [torch.zeros_like(w) for w in W]
    for t in range(6):
        gt = lact_token_grad(K[:, t], V[:, t], W)
        g = [a + eta[0, t] * b for a, b in zip(g, gt)]
    gen = torch.Generator().manual_seed(3)
    for _ in range(5):
        D = [torch.randn(w.shape, generator=gen, dtype=DT) for w in W]
        h = 1e-6
        fd = (loss(tuple(w + h * dd for w, dd in zip(W, D))) - loss(tuple(w - h * dd for w, dd in zip(W, D)))) / (2 * h)
        an = sum((gg * dd).sum() for gg, dd in zip(g, D))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (fd, an)


@pytest.mark.parametrize("apply", ["after", "before"])
@pytest.mark.parametrize("chunk", [1, 4, 16])
def test_scan_matches_library_reference(chunk, apply):
    Q, K, V, eta, W = _inputs(2, 16, 6, 12, seed=4 + chunk)
    Z, WT = scan_lact(Q, K, V, eta, W, chunk, apply=apply)
    Zr, WTr = _lib_scan(Q, K, V, eta, W, chunk, apply=apply)
    assert rel(Z, Zr) <= 1e-12
    for a, b in zip(WT, WTr):
        assert rel(a, b) <= 1e-12


def test_zero_step_closed_form():
    """eta = 0: no gradient, so every update only normalises; the first chunk's output is
    f(q; W0) when read out before the update and f(q; normalised W0) after it, and the final
    weights are W0 with unit-norm output units."""
    Q, K, V, eta, W = _inputs(2, 8, 5, 10, seed=9)
    eta = torch.zeros_like(eta)
    Wn = tuple(l2_normalize_units(w) for w in W)
    Z, WT = scan_lact(Q, K, V, eta, W, 4, apply="after")
    assert rel(Z, lact_apply(Q, Wn)) <= 1e-14
    for a, b in zip(WT, Wn):
        assert rel(a, b) <= 1e-14
    Zb, _ = scan_lact(Q, K, V, eta, W, 4, apply="before")
    assert rel(Zb[:, :4], lact_apply(Q[:, :4], W)) <= 1e-14
    assert rel(Zb[:, 4:], lact_apply(Q[:, 4:], Wn)) <= 1e-14


def test_updated_weights_have_unit_norm_units():
    Q, K, V, eta, W = _inputs(2, 12, 6, 10, seed=10)
    _, WT = scan_lact(Q, K, V, eta, W, 4)
    for w in WT:
        assert (w.norm(dim=-2) - 1.0).abs().max().item() <= 1e-13


def test_carry_is_bitwise():
    Q, K, V, eta, W = _inputs(2, 16, 6, 10, seed=11)
    Z, WT = scan_lact(Q, K, V, eta, W, 4)
    Za, Wa = scan_lact(Q[:, :8], K[:, :8], V[:, :8], eta[:, :8], W, 4)
    Zb, Wb = scan_lact(Q[:, 8:], K[:, 8:], V[:, 8:], eta[:, 8:], Wa, 4)
    assert torch.equal(torch.cat([Za, Zb], dim=1), Z)
    for a, b in zip(Wb, WT):
        assert torch.equal(a, b)


def test_step_descends_before_normalisation():
    """The unnormalised step W - g with a small eta lowers the chunk's summed loss (the sign of
    Eq. 4 and Eq. 8): a flipped sign or a dropped eta fails here."""
    Q, K, V, eta, W = _inputs(1, 8, 6, 12, seed=12)
    eta = 1e-3 * eta

    def chunk_loss(Wx):
        return sum(-(lact_apply(K[:, t], Wx)[0] @ V[0, t]) * eta[0, t] for t in range(8))

    g = [torch.zeros_like(w) for w in W]
    for t in range(8):
        g = [a + eta[0, t] * b for a, b in zip(g, lact_token_grad(K[:, t], V[:, t], W))]
    assert chunk_loss(tuple(w - gg for w, gg in zip(W, g))) < chunk_loss(W)
