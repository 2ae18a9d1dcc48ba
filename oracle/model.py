"""Plain, slow, fp64 numpy implementation of the d20 training step.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product never
imports this module.

What is computed, and where the pages state it (nanochat speedrun
walkthrough, lyylswood.com, "100 dollars, 8000 lines: a hand-built ChatGPT
clone"; sections named in English):

* the model is a Llama-like decoder-only Transformer, simplified, with ideas
  from modded-nanoGPT (introduction: the author's comment on the
  architecture);
* it is trained to predict the next token of packed rows (Pretraining);
* d20 has 20 layers, 1280 channels and 10 heads of dimension 128
  (Pretraining, the printed model summary);
* there are no biases and no RMSNorm parameters; embedding and unembedding
  are separate tensors, each optimised by AdamW (Pretraining, optimiser
  paragraph);
* the loss is also reported as bits per byte: per-token loss normalised by
  the bytes of each token (Pretraining, bits-per-byte paragraph).

Readings where the pages are silent (each listed in the design notes):
pre-norm blocks with one final norm before the unembedding; RMSNorm
y = x / sqrt(mean(x^2) + eps), eps = 1e-6; rotary positions on q and k with
adjacent pairs (2i, 2i+1), angle t * base^(-2i/Q), base 10000, positions
restarting at 0 in every row; attention scale 1/sqrt(Q) with a plain causal
mask over the packed row; full multi-head attention; MLP relu(h)^2 of width
4d; untied unembedding; mean cross-entropy over valid targets (target -1 is
ignored), taken as 0 when no target is valid; bits per byte =
sum(ce) / (ln 2 * sum(bytes[target])).

Rows are independent (attention never crosses a row), so everything runs
one row at a time and weight gradients are summed over rows in fp64.
No blocking, fusion or reordering: each step is the textbook formula, with
numpy's matmul as the only library primitive.
"""
from __future__ import annotations

import math
import numpy as np

LN2 = math.log(2.0)


# ---------------------------------------------------------------------------
# parameter-free RMSNorm
# ---------------------------------------------------------------------------
def rmsnorm(x: np.ndarray, eps: float):
    """y = x * r, r = (mean_j x_j^2 + eps)^(-1/2) over the last axis.

    Returns (y, r) with r of shape x.shape[:-1]."""
    ms = np.mean(x * x, axis=-1)
    r = 1.0 / np.sqrt(ms + eps)
    return x * r[..., None], r


def rmsnorm_bwd(y: np.ndarray, r: np.ndarray, dy: np.ndarray) -> np.ndarray:
    """Reverse mode of ``rmsnorm`` written with the saved output y = x*r:
    dx = r * (dy - y * mean_j(dy_j * y_j))."""
    return r[..., None] * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))


# ---------------------------------------------------------------------------
# rotary positions (adjacent pairs)
# ---------------------------------------------------------------------------
def rope_angles(T: int, Q: int, base: float) -> np.ndarray:
    """phi[t, i] = t * base^(-2i/Q) for t < T, i < Q/2 (float64)."""
    i = np.arange(Q // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / Q)
    t = np.arange(T, dtype=np.float64)
    return t[:, None] * theta[None, :]


def rope(x: np.ndarray, phi: np.ndarray, inverse: bool = False) -> np.ndarray:
    """Rotate each pair (x[2i], x[2i+1]) of every head by phi[t, i].

    x: [T, H, Q].  ``inverse`` rotates by -phi (the transpose, i.e. the
    reverse-mode map of the forward rotation)."""
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    if inverse:
        s = -s
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


# ---------------------------------------------------------------------------
# causal multi-head attention (dense, masked softmax)
# ---------------------------------------------------------------------------
def _softmax_rows(S: np.ndarray) -> np.ndarray:
    S = S - S.max(axis=-1, keepdims=True)
    P = np.exp(S)
    return P / P.sum(axis=-1, keepdims=True)


def _causal_probs(qh: np.ndarray, kh: np.ndarray) -> np.ndarray:
    T, Q = qh.shape
    S = (qh @ kh.T) / math.sqrt(Q)
    S[np.triu(np.ones((T, T), dtype=bool), 1)] = -np.inf   # key j > query t
    return _softmax_rows(S)


def causal_attention(q, k, v):
    """o[t,h] = sum_{j<=t} softmax_j(q[t,h].k[j,h] / sqrt(Q)) v[j,h].

    q, k, v: [T, H, Q] -> o [T, H, Q]."""
    T, H, Q = q.shape
    o = np.empty_like(q)
    for h in range(H):
        P = _causal_probs(q[:, h, :], k[:, h, :])
        o[:, h, :] = P @ v[:, h, :]
    return o


def causal_attention_bwd(q, k, v, do):
    """Reverse mode of ``causal_attention``; recomputes P.  The softmax
    Jacobian is applied as dS = P * (dP - sum_j P*dP)."""
    T, H, Q = q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    sc = 1.0 / math.sqrt(Q)
    for h in range(H):
        P = _causal_probs(q[:, h, :], k[:, h, :])
        doh = do[:, h, :]
        dv[:, h, :] = P.T @ doh
        dP = doh @ v[:, h, :].T
        dS = P * (dP - np.sum(P * dP, axis=-1, keepdims=True))
        dq[:, h, :] = (dS @ k[:, h, :]) * sc
        dk[:, h, :] = (dS.T @ q[:, h, :]) * sc
    return dq, dk, dv


# ---------------------------------------------------------------------------
# squared ReLU, cross-entropy, bits per byte
# ---------------------------------------------------------------------------
def relu2(h):
    return np.maximum(h, 0.0) ** 2


def relu2_grad(h):
    return 2.0 * np.maximum(h, 0.0)


def _logsumexp_rows(z):
    m = z.max(axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(z - m), axis=-1, keepdims=True)))[..., 0]


def cross_entropy(z, tgt):
    """ce[t] = logsumexp(z[t]) - z[t, tgt[t]]; 0 where tgt[t] < 0 (ignored)."""
    lse = _logsumexp_rows(z)
    valid = tgt >= 0
    zt = z[np.arange(z.shape[0]), np.where(valid, tgt, 0)]
    return np.where(valid, lse - zt, 0.0)


def cross_entropy_grad(z, tgt, scale):
    """d(sum_t scale_t ce[t])/dz = scale_t (softmax(z_t) - onehot(tgt_t));
    scale is one number or one per row; rows with an ignored target get 0."""
    dz = _softmax_rows(z)
    valid = tgt >= 0
    rows = np.nonzero(valid)[0]
    dz[rows, tgt[rows]] -= 1.0
    dz[~valid] = 0.0
    scale = np.asarray(scale, dtype=np.float64)
    return dz * (scale[:, None] if scale.ndim == 1 else scale)


def loss_bpb(ce, tgt, token_bytes):
    """(mean ce over valid targets in nats, bits per byte).

    bits per byte = sum(ce) / (ln 2 * sum of bytes of the target tokens)."""
    ce = np.asarray(ce, dtype=np.float64).ravel()
    tgt = np.asarray(tgt).ravel()
    valid = tgt >= 0
    s = float(np.sum(ce[valid]))
    nbytes = int(np.sum(np.asarray(token_bytes, dtype=np.int64)[tgt[valid]]))
    n = int(np.sum(valid))
    # no valid target: the mean over an empty set is taken as 0 (so is bpb)
    return (s / n if n else 0.0), (s / (LN2 * nbytes) if nbytes else 0.0)


# ---------------------------------------------------------------------------
# one pre-norm block
# ---------------------------------------------------------------------------

def sample_next(logits, temperature, top_k, u):
    """Next token from one row of logits, as the Engine samples (section
    Pretraining, the Engine paragraph): the largest logit when
    temperature == 0; otherwise p_i proportional to exp((z_i - max z) /
    temperature) over the top_k largest logits (all when top_k == 0; values
    tied with the k-th largest are kept), drawn by inverse CDF in token-id
    order: the first kept id whose running sum exceeds u * sum p
    (u in [0, 1); the last kept id if rounding leaves none)."""
    z = np.asarray(logits, dtype=np.float64)
    if temperature == 0:
        return int(np.argmax(z))
    keep = np.ones(z.shape, dtype=bool)
    if 0 < top_k < z.size:
        thr = np.sort(z)[::-1][top_k - 1]
        keep = z >= thr
    p = np.where(keep, np.exp((z - z.max()) / temperature), 0.0)
    c = np.cumsum(p)
    hit = np.nonzero((c > u * c[-1]) & keep)[0]
    return int(hit[0]) if hit.size else int(np.nonzero(keep)[0][-1])


def weighted_loss(ce, tgt, weights):
    """(sum over valid targets of w_t ce[t], that sum / n_valid); 0 when no
    target is valid."""
    ce = np.asarray(ce, dtype=np.float64).ravel()
    valid = np.asarray(tgt).ravel() >= 0
    w = np.asarray(weights, dtype=np.float64).ravel()
    s = float(np.sum(np.where(valid, w * ce, 0.0)))
    n = int(np.sum(valid))
    return s, (s / n if n else 0.0)

def block_forward(lp, x, cfg, phi):
    """x [T, d] -> y [T, d]; returns (y, cache)."""
    T, d = x.shape
    H, Q = cfg.n_head, cfg.head_dim
    a, r1 = rmsnorm(x, cfg.rms_eps)
    q = (a @ lp["Wq"].T).reshape(T, H, Q)
    k = (a @ lp["Wk"].T).reshape(T, H, Q)
    v = (a @ lp["Wv"].T).reshape(T, H, Q)
    qr, kr = rope(q, phi), rope(k, phi)
    o = causal_attention(qr, kr, v).reshape(T, d)
    x1 = x + o @ lp["Wo"].T
    m, r2 = rmsnorm(x1, cfg.rms_eps)
    h = m @ lp["W1"].T
    u = relu2(h)
    y = x1 + u @ lp["W2"].T
    cache = dict(a=a, r1=r1, qr=qr, kr=kr, v=v, o=o, m=m, r2=r2, h=h)
    return y, cache


def block_backward(lp, cache, g, cfg, phi, grads):
    """Given g = dL/dy, add the block's weight gradients into ``grads`` and
    return dL/dx."""
    T, d = g.shape
    H, Q = cfg.n_head, cfg.head_dim
    c = cache
    u = relu2(c["h"])
    grads["W2"] += g.T @ u
    du = g @ lp["W2"]
    dh = du * relu2_grad(c["h"])
    grads["W1"] += dh.T @ c["m"]
    dm = dh @ lp["W1"]
    g = g + rmsnorm_bwd(c["m"], c["r2"], dm)
    grads["Wo"] += g.T @ c["o"]
    do = (g @ lp["Wo"]).reshape(T, H, Q)
    dqr, dkr, dv = causal_attention_bwd(c["qr"], c["kr"], c["v"], do)
    dq = rope(dqr, phi, inverse=True).reshape(T, d)
    dk = rope(dkr, phi, inverse=True).reshape(T, d)
    dv = dv.reshape(T, d)
    grads["Wq"] += dq.T @ c["a"]
    grads["Wk"] += dk.T @ c["a"]
    grads["Wv"] += dv.T @ c["a"]
    da = dq @ lp["Wq"] + dk @ lp["Wk"] + dv @ lp["Wv"]
    return g + rmsnorm_bwd(c["a"], c["r1"], da)


# ---------------------------------------------------------------------------
# whole model, one row
# ---------------------------------------------------------------------------
def model_forward_row(params, idx_row, tgt_row, cfg, phi=None):
    """Forward over one packed row; returns (ce [T], cache)."""
    T = idx_row.shape[0]
    if phi is None:
        phi = rope_angles(T, cfg.head_dim, cfg.rope_base)
    x = params["E"][idx_row]
    caches = []
    for lp in params["layers"]:
        x, c = block_forward(lp, x, cfg, phi)
        caches.append(c)
    xf, rf = rmsnorm(x, cfg.rms_eps)
    z = xf @ params["U"].T
    ce = cross_entropy(z, tgt_row)
    return ce, dict(layers=caches, xf=xf, rf=rf, z=z, idx=idx_row, tgt=tgt_row, phi=phi)


def zero_grads(params):
    g = {"layers": [{k: np.zeros_like(v) for k, v in lp.items()} for lp in params["layers"]]}
    for k in ("E", "U"):
        if k in params:
            g[k] = np.zeros_like(params[k])
    return g


def model_backward_row(params, cache, cfg, scale, grads):
    """Add d(scale * sum_t ce[t])/dparams for one row into ``grads``."""
    dz = cross_entropy_grad(cache["z"], cache["tgt"], scale)
    grads["U"] += dz.T @ cache["xf"]
    dxf = dz @ params["U"]
    g = rmsnorm_bwd(cache["xf"], cache["rf"], dxf)
    for l in reversed(range(len(params["layers"]))):
        g = block_backward(params["layers"][l], cache["layers"][l], g, cfg,
                           cache["phi"], grads["layers"][l])
    np.add.at(grads["E"], cache["idx"], g)


def _to64(params):
    out = {"layers": [{k: np.asarray(v, dtype=np.float64) for k, v in lp.items()}
                      for lp in params["layers"]]}
    for k in ("E", "U"):
        if k in params:
            out[k] = np.asarray(params[k], dtype=np.float64)
    return out


def train_step(cfg, params, idx, tgt, token_bytes, want_grads=True, rows=None, token_weights=None):
    """One fwd(+bwd) step over the batch.

    params: {"E", "U", "layers": [{"Wq", "Wk", "Wv", "Wo", "W1", "W2"}]}
    idx, tgt: int [B, T].  Gradients are of the mean cross-entropy over all
    valid targets of the batch, or, with token_weights w [B, T], of
    sum_t w_t ce[t] / n_valid (the token-level weighted loss of the
    simplified GRPO, section Reinforcement learning: per-token advantage
    weights, normalised over tokens rather than sequences).  ``rows`` limits
    the work to the given row indices (the loss normalisation still counts
    the whole batch)."""
    p = _to64(params)
    idx = np.asarray(idx)
    tgt = np.asarray(tgt)
    B, T = idx.shape
    n_valid = int(np.sum(tgt >= 0))
    scale = 1.0 / n_valid if n_valid else 0.0     # no valid target: zero loss, zero gradient
    phi = rope_angles(T, cfg.head_dim, cfg.rope_base)
    ce = np.zeros((B, T), dtype=np.float64)
    grads = zero_grads(p) if want_grads else None
    for b in (range(B) if rows is None else rows):
        ce_b, cache = model_forward_row(p, idx[b], tgt[b], cfg, phi)
        ce[b] = ce_b
        if want_grads:
            row_scale = scale if token_weights is None else scale * np.asarray(token_weights[b], dtype=np.float64)
            model_backward_row(p, cache, cfg, row_scale, grads)
        del cache
    out = dict(ce=ce, grads=grads)
    if rows is None:
        out["loss"], out["bpb"] = loss_bpb(ce, tgt, token_bytes)
    return out


def block_step(cfg, lp, x, dy, rows=None):
    """Single block: y = block(x) and its VJP with dy, summed over rows.

    x, dy: [B, T, d].  Returns dict(y, dx, grads)."""
    lp = {k: np.asarray(v, dtype=np.float64) for k, v in lp.items()}
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    B, T, d = x.shape
    phi = rope_angles(T, cfg.head_dim, cfg.rope_base)
    y = np.zeros_like(x)
    dx = np.zeros_like(x)
    grads = {k: np.zeros_like(v) for k, v in lp.items()}
    for b in (range(B) if rows is None else rows):
        y[b], c = block_forward(lp, x[b], cfg, phi)
        dx[b] = block_backward(lp, c, dy[b], cfg, phi, grads)
    return dict(y=y, dx=dx, grads=grads)
