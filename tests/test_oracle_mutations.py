"""The oracle's pins against planted mistakes (CPU only).

Each case replaces one function of the oracle with a copy carrying one plausible
mistake, then runs a fixed set of pins from test_oracle_pins.py: at least one of
them must fail. Without a mistake all of them pass. The mistakes are the ones a
re-derivation of the scan ("Test-Time Training(TTT)과 LLM 메모리", section "TTT
layer", Eq. 2/4/5; the mini-batch rule of the E2E paper review, section 2.3, Eq. 5)
most easily gets wrong: a dropped LayerNorm-backward term, a missing factor 2 of the
squared loss, the residual left out of the loss, the unbiased variance, epsilon
outside the square root, an exclusive prefix for the output, and the gradient taken
at the running weights instead of the chunk-start weights."""
import pytest
import torch

import oracle.ttt_oracle as O
import test_oracle_pins as P


# ---------------------------------------------------------------------------
# The planted mistakes (each a copy of one oracle function with one change)
# ---------------------------------------------------------------------------

def _grad_variant(drop_ln_term=False, no_factor2=False, no_residual=False):
    def token_loss_and_grad(x, y, W, gamma, beta, cfg):
        z, cache = O.inner_forward(x, W, cfg)
        if cfg.layer_norm:
            ln_out, xhat, sigma = O.layer_norm(z, gamma, beta, cfg.ln_eps)
        else:
            ln_out = z
        pred = x + ln_out if (cfg.residual and not no_residual) else ln_out
        r = pred - y
        loss = (r * r).sum(dim=-1)
        f2 = 1.0 if no_factor2 else 2.0
        if cfg.layer_norm:
            gg = f2 * r * gamma
            delta2 = gg - gg.mean(dim=-1, keepdim=True)
            if not drop_ln_term:
                delta2 = delta2 - xhat * (gg * xhat).mean(dim=-1, keepdim=True)
            delta2 = delta2 / sigma
        else:
            delta2 = f2 * r
        if cfg.kind == "mlp":
            W1, W2 = W
            a, c = cache
            gW2 = torch.einsum("nh,nd->nhd", c, delta2)
            delta1 = torch.einsum("nd,nhd->nh", delta2, W2) * O.gelu_prime(a, cfg.gelu)
            gW1 = torch.einsum("nd,nh->ndh", x, delta1)
            return loss, (gW1, gW2)
        return loss, (torch.einsum("nd,ne->nde", x, delta2),)
    return token_loss_and_grad


def _ln_variant(unbiased=False, eps_outside=False):
    def layer_norm(z, gamma, beta, eps):
        mu = z.mean(dim=-1, keepdim=True)
        n = z.shape[-1]
        var = ((z - mu) ** 2).sum(dim=-1, keepdim=True) / (n - 1 if unbiased else n)
        sigma = torch.sqrt(var) + eps if eps_outside else torch.sqrt(var + eps)
        xhat = (z - mu) / sigma
        return gamma * xhat + beta, xhat, sigma
    return layer_norm


def _scan_variant(exclusive=False, running_grad=False):
    def scan(Q, K, V, eta, W0, gamma, beta, cfg):
        N, T, d = Q.shape
        b = cfg.chunk
        W = tuple(W0)
        Z, losses = [], []
        for i in range(T // b):
            W_start = W
            P_ = tuple(torch.zeros_like(w) for w in W_start)
            for t in range(i * b, (i + 1) * b):
                W_at = tuple(ws - p for ws, p in zip(W_start, P_)) if running_grad else W_start
                loss, grads = O.token_loss_and_grad(K[:, t], V[:, t], W_at, gamma, beta, cfg)
                step = cfg.eta_scale * eta[:, t].reshape(N, 1, 1)
                P_before = P_
                P_ = tuple(p + step * gw for p, gw in zip(P_, grads))
                W_t = tuple(ws - p for ws, p in zip(W_start, P_before if exclusive else P_))
                Z.append(O.f_apply(Q[:, t], W_t, gamma, beta, cfg))
                losses.append(loss)
            W = tuple(ws - p for ws, p in zip(W_start, P_))
        return torch.stack(Z, dim=1), W, torch.stack(losses, dim=1)
    return scan


MUTATIONS = {
    "dropped LN-backward term": {"token_loss_and_grad": _grad_variant(drop_ln_term=True)},
    "missing factor 2": {"token_loss_and_grad": _grad_variant(no_factor2=True)},
    "no residual in the loss": {"token_loss_and_grad": _grad_variant(no_residual=True)},
    "unbiased variance": {"layer_norm": _ln_variant(unbiased=True)},
    "epsilon outside the square root": {"layer_norm": _ln_variant(eps_outside=True)},
    "exclusive prefix": {"scan": _scan_variant(exclusive=True)},
    "gradient at the running weights": {"scan": _scan_variant(running_grad=True)},
}

# The pins run against every mutation (a subset of test_oracle_pins.py, small sizes).
PINS = {
    "token gradient vs finite differences": lambda: P.test_token_grad_central_finite_differences("mlp"),
    "token gradient vs library autograd": lambda: P.test_token_grad_matches_autograd_of_library_layer("mlp", "erf"),
    "LayerNorm scale invariance": lambda: P.test_layernorm_scale_invariance_orthogonality("mlp"),
    "b = 1 vs sequential loop": lambda: P.test_b1_equals_sequential_loop("mlp"),
    "mini-batch vs library autograd": lambda: P.test_minibatch_matches_autograd_reference("mlp", "erf"),
    "Theorem 1 golden": P.test_golden_theorem1_linear_attention,
    "delta rule golden": P.test_golden_delta_rule,
}


def _patch(monkeypatch, repl):
    for name, fn in repl.items():
        monkeypatch.setattr(O, name, fn)
        if hasattr(P, name):
            monkeypatch.setattr(P, name, fn)


def _failing_pins():
    failed = []
    for name, pin in PINS.items():
        try:
            pin()
        except AssertionError:
            failed.append(name)
    return failed


def test_pins_pass_without_a_mistake():
    assert _failing_pins() == []


@pytest.mark.parametrize("mutation", list(MUTATIONS))
def test_each_planted_mistake_fails_a_pin(mutation, monkeypatch):
    _patch(monkeypatch, MUTATIONS[mutation])
    failed = _failing_pins()
    assert failed, f"no pin caught: {mutation}"
