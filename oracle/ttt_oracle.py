"""Plain fp64 CPU oracle for the TTT-Linear / TTT-MLP mini-batch inner-loop scan.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this module. The product path (the HIP library and its
Python binding) never calls it, and it shares no code with that path.

What it computes (sources, by page title and section):

* "Test-Time Training(TTT)과 LLM 메모리" (juhoplayground), section "TTT layer":
  the layer keeps fast weights W as its hidden state, takes the self-supervised
  loss l(W; x_t) = || f(theta_K x_t; W) - theta_V x_t ||^2 (Eq. 4), takes the step
  W_t = W_{t-1} - eta * grad l (Eq. 2) and outputs z_t = f(theta_Q x_t; W_t) (Eq. 5).
  The conceptual loop given there updates W *before* producing z_t.
  TTT-Linear: f is linear with a square W; TTT-MLP: a two-layer MLP with a 4x
  hidden width and GELU. Both include LayerNorm and a residual. The practical
  devices are mini-batch TTT with b = 16, the dual form, a learnable W0 and a
  learnable per-token eta.
* Same page, section "재현성과 공개 구현": the stabilising form f(x) = x + LN(f_res(x)).
* "LLM : 빠른 논문 리뷰 : End-to-End Test-Time Training for Long Context", section 2.4.2,
  Eq. 9 (the simplified output rule, an option here): the output reuses the key-side
  prediction g(theta_K x_t; W_{t-1}) instead of evaluating f again on theta_Q x_t with the
  updated weights. In the mini-batch scan the gradient of token t is taken at the chunk's
  start weights, so the plain reading is z_t = f(K_t; W_start); with b = 1 that is W_{t-1}.
* "LLM : 빠른 논문 리뷰 : End-to-End Test-Time Training for Long Context"
  (aiflower), section 2.3, Eq. 5: in a mini-batch all gradients are taken at the
  weights the mini-batch started from, and W is carried into the next mini-batch.

Plain reading of open points (each also listed in the design notes):
* eta is applied as given per token, as a plain (un-normalised) sum; eta_scale
  multiplies every eta (1/b gives the 1/b form written in Eq. 5 of the E2E paper).
* Inside a chunk, z_t uses W_t = W_start - sum_{s<=t} eta_s grad l_s(W_start),
  i.e. token t's own step is included (update before output).
* LayerNorm uses the biased variance and sigma = sqrt(var + eps).
* gamma, beta (the LayerNorm affine) are outer-loop parameters, fixed in the scan.
* No biases inside the fast MLP / linear map.
* GELU is the exact erf form by default; the tanh form is an option.

Layout (row vectors): Q, K, V are [N, T, d] with N = independent (batch, head)
pairs. TTT-MLP: W1 [N, d, h], W2 [N, h, d], g(x) = GELU(x W1) W2. TTT-Linear:
W [N, d, d], g(x) = x W. eta is [N, T]; gamma, beta are [N, d].

The gradient of one token's loss is derived by hand below. It is written with
ordinary differentiable torch ops, so torch.autograd can differentiate the whole
scan again (gradients of gradients) for the outer-loop backward oracle.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)
_TANH_C = math.sqrt(2.0 / math.pi)
_TANH_A = 0.044715


@dataclass(frozen=True)
class OracleConfig:
    """Static description of one scan.

    kind: "mlp" or "linear".
    chunk: mini-batch size b (T must be a multiple of it).
    ln_eps: epsilon inside the LayerNorm square root.
    gelu: "erf" (exact) or "tanh".
    eta_scale: multiplies every per-token eta.
    layer_norm / residual: both True for the layer as defined; switching both off
        gives the plain map f(x) = g(x) used by the attention-equivalence checks.
    output: "query" (Eq. 5/8: z_t = f(Q_t; W_t)) or "key" (Eq. 9 of the E2E review:
        z_t = f(K_t; W_start), the prediction the token's loss is taken on).
    """

    kind: str = "mlp"
    chunk: int = 16
    ln_eps: float = 1e-6
    gelu: str = "erf"
    eta_scale: float = 1.0
    layer_norm: bool = True
    residual: bool = True
    output: str = "query"


# ----------------------------------------------------------------------------
# Elementwise pieces
# ----------------------------------------------------------------------------

def gelu(x: torch.Tensor, kind: str = "erf") -> torch.Tensor:
    """GELU(x) = x * Phi(x) (erf form) or the usual tanh approximation."""
    if kind == "erf":
        return 0.5 * x * (1.0 + torch.erf(x / _SQRT2))
    if kind == "tanh":
        return 0.5 * x * (1.0 + torch.tanh(_TANH_C * (x + _TANH_A * x ** 3)))
    raise ValueError(kind)


def gelu_prime(x: torch.Tensor, kind: str = "erf") -> torch.Tensor:
    """d GELU / dx. erf form: Phi(x) + x * phi(x)."""
    if kind == "erf":
        cdf = 0.5 * (1.0 + torch.erf(x / _SQRT2))
        pdf = torch.exp(-0.5 * x * x) * _INV_SQRT_2PI
        return cdf + x * pdf
    if kind == "tanh":
        u = _TANH_C * (x + _TANH_A * x ** 3)
        th = torch.tanh(u)
        du = _TANH_C * (1.0 + 3.0 * _TANH_A * x * x)
        return 0.5 * (1.0 + th) + 0.5 * x * (1.0 - th * th) * du
    raise ValueError(kind)


# ----------------------------------------------------------------------------
# The fast-weight map f and one token's loss gradient
# ----------------------------------------------------------------------------

def inner_forward(x: torch.Tensor, W: tuple, cfg: OracleConfig):
    """g(x; W) for row vectors x [N, d]. Returns (g, cache)."""
    if cfg.kind == "mlp":
        W1, W2 = W
        a = torch.einsum("nd,ndh->nh", x, W1)
        c = gelu(a, cfg.gelu)
        g = torch.einsum("nh,nhd->nd", c, W2)
        return g, (a, c)
    (Wl,) = W
    return torch.einsum("nd,nde->ne", x, Wl), None


def layer_norm(z: torch.Tensor, gamma, beta, eps: float):
    """LayerNorm over the last axis, biased variance. Returns (out, xhat, sigma)."""
    mu = z.mean(dim=-1, keepdim=True)
    var = ((z - mu) ** 2).mean(dim=-1, keepdim=True)
    sigma = torch.sqrt(var + eps)
    xhat = (z - mu) / sigma
    return gamma * xhat + beta, xhat, sigma


def f_apply(x: torch.Tensor, W: tuple, gamma, beta, cfg: OracleConfig) -> torch.Tensor:
    """f(x; W) = x + LN(g(x; W)) (or the plain g(x; W) when LN/residual are off)."""
    g, _ = inner_forward(x, W, cfg)
    out = layer_norm(g, gamma, beta, cfg.ln_eps)[0] if cfg.layer_norm else g
    return x + out if cfg.residual else out


def token_loss_and_grad(x, y, W: tuple, gamma, beta, cfg: OracleConfig):
    """l = ||f(x;W) - y||^2 and its gradient w.r.t. each fast weight.

    Hand derivation (row vectors, per head):
      z = g(x;W);  xhat = (z - mu)/sigma;  r = x + gamma*xhat + beta - y;  l = sum r^2
      dl/dxhat = 2 r * gamma =: gg
      dl/dz = (gg - mean(gg) - xhat * mean(gg * xhat)) / sigma =: delta2
      MLP:    dl/dW2 = c^T delta2,   delta1 = (delta2 W2^T) * GELU'(a),  dl/dW1 = x^T delta1
      Linear: dl/dW  = x^T delta2
    The loss carries no 1/2 factor (Eq. 4 is the plain squared norm).
    """
    z, cache = inner_forward(x, W, cfg)
    if cfg.layer_norm:
        ln_out, xhat, sigma = layer_norm(z, gamma, beta, cfg.ln_eps)
    else:
        ln_out = z
    pred = x + ln_out if cfg.residual else ln_out
    r = pred - y
    loss = (r * r).sum(dim=-1)
    if cfg.layer_norm:
        gg = 2.0 * r * gamma
        delta2 = (gg - gg.mean(dim=-1, keepdim=True)
                  - xhat * (gg * xhat).mean(dim=-1, keepdim=True)) / sigma
    else:
        delta2 = 2.0 * r
    if cfg.kind == "mlp":
        W1, W2 = W
        a, c = cache
        gW2 = torch.einsum("nh,nd->nhd", c, delta2)
        delta1 = torch.einsum("nd,nhd->nh", delta2, W2) * gelu_prime(a, cfg.gelu)
        gW1 = torch.einsum("nd,nh->ndh", x, delta1)
        return loss, (gW1, gW2)
    return loss, (torch.einsum("nd,ne->nde", x, delta2),)


# ----------------------------------------------------------------------------
# The scan
# ----------------------------------------------------------------------------

def scan(Q, K, V, eta, W0: tuple, gamma, beta, cfg: OracleConfig):
    """Mini-batch TTT scan, primal and token by token.

    For chunk i (tokens (i-1)b+1 .. ib), with W_start the weights carried in:
      for each token t of the chunk, in order:
        grad_t = grad l_t(W_start)                     (all gradients at the chunk start)
        P     += eta_scale * eta_t * grad_t            (running sum, t included)
        W_t    = W_start - P                           (materialised)
        z_t    = f(Q_t; W_t)         (output "key": z_t = f(K_t; W_start))
      carry W_start <- W_start - P.
    Returns Z [N, T, d], the final weights (tuple) and the per-token loss [N, T]
    l_t(W_start) (the reconstruction loss at the weights the gradient is taken at).
    """
    N, T, d = Q.shape
    b = cfg.chunk
    if T % b != 0:
        raise ValueError("T must be a multiple of the chunk size")
    W = tuple(w for w in W0)
    Z = []
    losses = []
    for i in range(T // b):
        W_start = W
        P = tuple(torch.zeros_like(w) for w in W_start)
        for t in range(i * b, (i + 1) * b):
            loss, grads = token_loss_and_grad(K[:, t], V[:, t], W_start, gamma, beta, cfg)
            step = cfg.eta_scale * eta[:, t].reshape(N, 1, 1)
            P = tuple(p + step * gw for p, gw in zip(P, grads))
            if cfg.output == "key":
                Z.append(f_apply(K[:, t], W_start, gamma, beta, cfg))
            elif cfg.output == "query":
                W_t = tuple(ws - p for ws, p in zip(W_start, P))
                Z.append(f_apply(Q[:, t], W_t, gamma, beta, cfg))
            else:
                raise ValueError(cfg.output)
            losses.append(loss)
        W = tuple(ws - p for ws, p in zip(W_start, P))
    return torch.stack(Z, dim=1), W, torch.stack(losses, dim=1)


def scan_momentum(Q, K, V, theta, mom, alpha, W0: tuple, S0: tuple | None, gamma, beta,
                  cfg: OracleConfig):
    """Mini-batch scan with momentum and a forget gate, primal and token by token.

    "Test-Time Training(TTT)과 LLM 메모리", section "Titans와 Miras", Eq. 14 and Eq. 13:
      S_t = eta_t S_{t-1} - theta_t grad l(M_{t-1}; x_t)     (momentum; eta here is `mom`)
      M_t = (1 - alpha_t) M_{t-1} + S_t                      (forget gate)
    with the mini-batch rule of the base scan (E2E paper review, section 2.3, Eq. 5): inside a
    chunk every gradient is taken at the memory the chunk started from, so for b = 1 this is
    the per-token rule as written. The output is z_t = f(Q_t; M_t), after token t's update.
    theta (the step size, times cfg.eta_scale), mom and alpha are [N, T]; S0 is the momentum
    carried in (zeros when None). M and S are both carried across chunks. With mom = 0 and
    alpha = 0 this is the base scan with eta = theta.
    Returns Z [N, T, d], the final memory M_T and momentum S_T (tuples) and the loss [N, T].
    """
    N, T, d = Q.shape
    b = cfg.chunk
    if T % b != 0:
        raise ValueError("T must be a multiple of the chunk size")
    if cfg.output != "query":
        raise ValueError("the momentum scan has the query output only")
    M = tuple(w for w in W0)
    S = tuple(torch.zeros_like(w) for w in W0) if S0 is None else tuple(s for s in S0)
    Z, losses = [], []
    for i in range(T // b):
        M_start = M
        for t in range(i * b, (i + 1) * b):
            loss, grads = token_loss_and_grad(K[:, t], V[:, t], M_start, gamma, beta, cfg)
            th = (cfg.eta_scale * theta[:, t]).reshape(N, 1, 1)
            mo = mom[:, t].reshape(N, 1, 1)
            keep = (1.0 - alpha[:, t]).reshape(N, 1, 1)
            S = tuple(mo * sv - th * gw for sv, gw in zip(S, grads))
            M = tuple(keep * m + sv for m, sv in zip(M, S))
            Z.append(f_apply(Q[:, t], M, gamma, beta, cfg))
            losses.append(loss)
    return torch.stack(Z, dim=1), M, S, torch.stack(losses, dim=1)


def scan_outer_grads(Q, K, V, eta, W0: tuple, gamma, beta, cfg: OracleConfig,
                     dZ, dW_T: tuple | None = None):
    """Outer-loop backward by automatic differentiation through the scan.

    L = sum(dZ * Z) + sum_k sum(dW_T[k] * W_T[k]). Because the scan's update is
    itself a gradient, differentiating L w.r.t. W0, Q, K, V and eta takes gradients
    of gradients (the outer loop of "LLM : 빠른 논문 리뷰 : End-to-End Test-Time
    Training for Long Context", section 2.2). Returns a dict of fp64 tensors:
    dQ, dK, dV, deta, dW0 (tuple), dgamma, dbeta.
    """
    leaves = [t.detach().clone().requires_grad_(True) for t in (Q, K, V, eta, gamma, beta)]
    Wl = [w.detach().clone().requires_grad_(True) for w in W0]
    q, k, v, e, gm, bt = leaves
    Z, W_T, _ = scan(q, k, v, e, tuple(Wl), gm, bt, cfg)
    L = (Z * dZ).sum()
    if dW_T is not None:
        for w, dw in zip(W_T, dW_T):
            L = L + (w * dw).sum()
    # (with the Eq. 9 output rule Q is not read: its gradient is zero)
    grads = torch.autograd.grad(L, leaves + Wl, allow_unused=True)
    grads = [torch.zeros_like(x) if gr is None else gr for gr, x in zip(grads, leaves + Wl)]
    return {
        "dQ": grads[0], "dK": grads[1], "dV": grads[2], "deta": grads[3],
        "dgamma": grads[4], "dbeta": grads[5], "dW0": tuple(grads[6:]),
    }


# ----------------------------------------------------------------------------
# Large-chunk TTT with SwiGLU fast weights and L2-normalised weights (LaCT)
# ----------------------------------------------------------------------------

def silu(x: torch.Tensor) -> torch.Tensor:
    """SiLU(x) = x * sigmoid(x)."""
    return x * torch.sigmoid(x)


def silu_prime(x: torch.Tensor) -> torch.Tensor:
    """d SiLU / dx = sigmoid(x) * (1 + x * (1 - sigmoid(x)))."""
    s = torch.sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


def lact_apply(x: torch.Tensor, W: tuple) -> torch.Tensor:
    """f_W(x) = (SiLU(x W1) * (x W3)) W2 for row vectors x [N, d] (or [N, n, d]):
    "Test-Time Training(TTT)과 LLM 메모리", section "LaCT", Eq. 6, f_W(x) = W2[SiLU(W1 x) o (W3 x)],
    with the page's column-vector weights stored transposed: W1, W3 [N, d, h], W2 [N, h, d]."""
    W1, W2, W3 = W
    if x.dim() == 2:
        a = torch.einsum("nd,ndh->nh", x, W1)
        c = torch.einsum("nd,ndh->nh", x, W3)
        return torch.einsum("nh,nhd->nd", silu(a) * c, W2)
    a = torch.einsum("ntd,ndh->nth", x, W1)
    c = torch.einsum("ntd,ndh->nth", x, W3)
    return torch.einsum("nth,nhd->ntd", silu(a) * c, W2)


def lact_token_grad(k: torch.Tensor, v: torch.Tensor, W: tuple):
    """Gradient of the token loss l = -f_W(k) . v (same page and section, Eq. 7) with respect to
    (W1, W2, W3), for row vectors k, v [N, d]. Hand derivation:
      a = k W1, c = k W3, s = SiLU(a), u = s * c, f = u W2, l = -f . v
      dl/dW2 = -u^T v;  gu = dl/du = -v W2^T
      dl/dW3 = k^T (gu * s);  dl/dW1 = k^T (gu * c * SiLU'(a))."""
    W1, W2, W3 = W
    a = torch.einsum("nd,ndh->nh", k, W1)
    c = torch.einsum("nd,ndh->nh", k, W3)
    s = silu(a)
    u = s * c
    gW2 = -torch.einsum("nh,nd->nhd", u, v)
    gu = -torch.einsum("nd,nhd->nh", v, W2)
    gW3 = torch.einsum("nd,nh->ndh", k, gu * s)
    gW1 = torch.einsum("nd,nh->ndh", k, gu * c * silu_prime(a))
    return gW1, gW2, gW3


def l2_normalize_units(W: torch.Tensor) -> torch.Tensor:
    """Each output unit's weight vector scaled to unit L2 norm. With the row-vector storage
    [N, inputs, outputs] that is every column (a row of the page's column-vector matrix)."""
    return W / W.norm(dim=-2, keepdim=True)


def scan_lact(Q, K, V, eta, W0: tuple, chunk: int, eta_scale: float = 1.0, apply: str = "after"):
    """Large-chunk TTT layer of "Test-Time Training(TTT)과 LLM 메모리", section "LaCT": per chunk of
    b tokens, the gradient g = grad_W sum_i eta_i l(f_W(k_i), v_i) of the chunk's summed loss at
    the chunk-start weights (Eq. 4 with the loss of Eq. 7), the update W <- L2-Normalize(W - g)
    (Eq. 8, each weight matrix per output unit), and the output o = f_W(q) (Eq. 2).

    apply = "after": a chunk's tokens are read out with the weights after that chunk's update
    (the order the section lists the steps in); "before": with the weights the chunk started from.
    Q, K, V [N, T, d], eta [N, T]; W0 = (W1 [N, d, h], W2 [N, h, d], W3 [N, d, h]).
    Returns Z [N, T, d] and the final weights."""
    N, T, d = Q.shape
    if T % chunk != 0:
        raise ValueError("T must be a multiple of the chunk size")
    if apply not in ("after", "before"):
        raise ValueError(apply)
    W = tuple(w for w in W0)
    Z = []
    for i in range(T // chunk):
        sl = slice(i * chunk, (i + 1) * chunk)
        G = tuple(torch.zeros_like(w) for w in W)
        for t in range(i * chunk, (i + 1) * chunk):
            g = lact_token_grad(K[:, t], V[:, t], W)
            step = eta_scale * eta[:, t].reshape(N, 1, 1)
            G = tuple(acc + step * gw for acc, gw in zip(G, g))
        W_new = tuple(l2_normalize_units(w - gw) for w, gw in zip(W, G))
        Z.append(lact_apply(Q[:, sl], W_new if apply == "after" else W))
        W = W_new
    return torch.cat(Z, dim=1), W
