"""Helpers for the GPU parity tests: host <-> device copies of fp32 / bf16
storage and the error metrics the tolerances are stated in."""
import numpy as np

import synthdata


def dev(arr, dtype="f32"):
    """numpy array -> CUDA tensor holding fp32 or bf16 storage (bf16 as raw
    int16 bits; values must already be bf16-exact to round-trip)."""
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype in (np.int32, np.int64):
        return torch.from_numpy(a.astype(np.int32)).cuda()
    if dtype == "bf16":
        bits = synthdata.f32_to_bf16_bits(a.astype(np.float32))
        return torch.from_numpy(bits.view(np.int16)).cuda()
    return torch.from_numpy(a.astype(np.float32)).cuda()


def host(t, dtype="f32"):
    """CUDA tensor of fp32 / bf16 storage -> float64 numpy."""
    a = t.detach().cpu().numpy()
    if dtype == "bf16":
        return synthdata.bf16_bits_to_f32(a.view(np.uint16)).astype(np.float64)
    return a.astype(np.float64)


def empty(shape, dtype="f32"):
    import torch
    tdt = {"f32": torch.float32, "bf16": torch.int16, "i32": torch.int32, "f64": torch.float64}[dtype]
    return torch.empty(shape, dtype=tdt, device="cuda")


def zeros(shape, dtype="f32"):
    t = empty(shape, dtype)
    t.zero_()
    return t


def max_rel_err(got, want):
    """max_i |got_i - want_i| / max_i |want_i| (the fp32-mode measure)."""
    got = np.asarray(got, dtype=np.float64).ravel()
    want = np.asarray(want, dtype=np.float64).ravel()
    den = np.max(np.abs(want))
    return float(np.max(np.abs(got - want)) / (den if den > 0 else 1.0))


def cosine(got, want):
    got = np.asarray(got, dtype=np.float64).ravel()
    want = np.asarray(want, dtype=np.float64).ravel()
    ng, nw = np.linalg.norm(got), np.linalg.norm(want)
    if ng == 0 and nw == 0:
        return 1.0
    return float(got @ want / (ng * nw))


def flat_tensors(cfg, flat_or_dict):
    """Yield (name, layer, array) over the flat layout, from a flat vector
    or an oracle gradient dict."""
    for name, layer, r, c, off in synthdata.param_layout(cfg):
        if isinstance(flat_or_dict, dict):
            a = flat_or_dict[name] if layer < 0 else flat_or_dict["layers"][layer][name]
        else:
            a = flat_or_dict[off:off + r * c].reshape(r, c)
        yield name, layer, a


def newton_schulz_bf16(G, steps, coeffs, eps=1e-7):
    """Error model of the Newton-Schulz iteration run with bf16 operands and
    fp32 accumulation: the oracle's iteration (oracle/optim.py) with every
    product's result rounded to bf16 where the library stores it (X, A,
    B = c A A + b A, X' = B X + a X).  It serves only to size the
    tolerance: on rank-deficient inputs (real gradients of a few hundred
    tokens) bf16 rounding alone moves the result well past a fixed cosine
    bar, and this says by how much for the input at hand."""
    a, b, c = coeffs
    r32 = lambda x: synthdata.bf16_bits_to_f32(synthdata.f32_to_bf16_bits(np.asarray(x, np.float32))).astype(np.float64)
    tall = G.shape[0] > G.shape[1]
    X = G.T if tall else G
    X = r32(X / (np.linalg.norm(X) + eps))
    for _ in range(steps):
        A = r32(X @ X.T)
        B = r32(c * (A @ A.T) + b * A)
        X = r32(B @ X + a * X)
    return X.T if tall else X


def logits_bf16_storage(cfg, p64, tokens):
    """Error model of the bf16 forward, used only to size the decode
    tolerance: the oracle's components (oracle/model.py) composed as the
    library stores activations -- the residual stream, both norm outputs, q
    and k after rotation, v, the attention output, relu(h)^2 and the final
    norm rounded to bf16 where the library writes them; weights are the
    same bf16 values; every product is exact (fp64).  The fp32 logits of
    every position, [T][V]."""
    import oracle
    r = lambda x: synthdata.round_to_bf16(np.asarray(x, np.float32)).astype(np.float64)
    tokens = np.asarray(tokens)
    T, H, Q = len(tokens), cfg.n_head, cfg.head_dim
    phi = oracle.rope_angles(T, Q, cfg.rope_base)
    x = p64["E"][tokens]
    for lp in p64["layers"]:
        a = r(oracle.rmsnorm(x, cfg.rms_eps)[0])
        q = r(oracle.rope((a @ lp["Wq"].T).reshape(T, H, Q), phi))
        k = r(oracle.rope((a @ lp["Wk"].T).reshape(T, H, Q), phi))
        v = r((a @ lp["Wv"].T).reshape(T, H, Q))
        o = r(oracle.causal_attention(q, k, v).reshape(T, -1))
        x = r(x + o @ lp["Wo"].T)
        m = r(oracle.rmsnorm(x, cfg.rms_eps)[0])
        u = r(oracle.relu2(m @ lp["W1"].T))
        x = r(x + u @ lp["W2"].T)
    xf = r(oracle.rmsnorm(x, cfg.rms_eps)[0])
    return xf @ p64["U"].T


# ---------------------------------------------------------------------------
# Rounding model of the matrix-core attention kernels (one head).  The
# kernels' arithmetic is written out step by step with every rounding the
# kernels make: scores accumulated to fp32, the log2-scaled exponent formed
# by one fused multiply-add in fp32, the lazily raised reference maximum
# (raised for all 32 rows of a wave when any row's 64-key tile maximum
# passes it by more than 8), the exponentials' bf16 rounding where they
# enter a product (P for PV and P^T dO, dS for dS K and dS^T Q), fp32 row
# sums, and the final bf16 stores.  What it leaves out is the order of the
# fp32 sums and the hardware exp2 / log2 / reciprocal error -- a few fp32
# ulps each -- so a kernel that follows these steps reproduces the model's
# bf16 outputs bit for bit except where such an ulp moves a value across a
# bf16 rounding boundary (about one rounding in 2^13).
# ---------------------------------------------------------------------------
_F32 = np.float32
_SCALE = _F32(0.08838834764831845)                      # 1 / sqrt(128)
_SCALE_LOG2 = _F32(_F32(1.4426950408889634) * _SCALE)   # log2(e) / sqrt(128), as the kernels form it


def _bf16(x):
    return synthdata.round_to_bf16(np.asarray(x, _F32)).astype(np.float64)


def attention_fwd_rounding_model(q, k, v):
    """Forward of one head: q, k, v [T][128] (bf16 values, T a multiple of
    64) -> (bf16 output [T][128] as float64, fp32 log-sum-exp [T])."""
    T, Q = q.shape
    S = (q @ k.T).astype(_F32)
    out = np.zeros((T, Q))
    lse = np.zeros(T, _F32)
    for w0 in range(0, T, 32):
        rows = np.arange(w0, min(w0 + 32, T))
        last = (w0 + 31) // 64                      # the wave's diagonal tile
        m = np.full(len(rows), -np.inf, _F32)
        l = np.zeros(len(rows))
        o = np.zeros((len(rows), Q))
        for jt in range(last + 1):
            j0, j1 = jt * 64, min(jt * 64 + 64, T)
            s = S[rows[0]:rows[-1] + 1, j0:j1].copy()
            s[np.arange(j0, j1)[None, :] > rows[:, None]] = -np.inf
            mx = (s.max(axis=1) * _SCALE_LOG2).astype(_F32)
            if np.any(mx > m + _F32(8)):
                mn = np.maximum(m, mx)
                alpha = np.exp2((m - mn).astype(np.float64))
                l, o, m = l * alpha, o * alpha[:, None], mn
            x = (s.astype(np.float64) * np.float64(_SCALE_LOG2) - m[:, None].astype(np.float64)).astype(_F32)
            p = np.exp2(x.astype(np.float64)).astype(_F32)
            l = l + p.astype(np.float64).sum(axis=1)
            o = o + _bf16(p) @ v[j0:j1]
        lf = l.astype(_F32)
        inv = (_F32(1) / lf).astype(_F32)
        out[rows] = _bf16(o.astype(_F32) * inv[:, None])
        lse[rows] = ((m + np.log2(lf)).astype(_F32) * _F32(0.69314718055994531)).astype(_F32)
    return out, lse


def attention_bwd_rounding_model(q, k, v, o, lse, do):
    """Backward of one head from the model's own forward (o bf16 values,
    lse fp32) and dO (bf16 values): (dq, dk, dv) as the kernels store them
    (bf16, before any rotary rotation) as float64."""
    T = q.shape[0]
    delta = (do * o).sum(axis=1).astype(_F32)
    lse2 = (lse.astype(_F32) * _F32(1.4426950408889634)).astype(_F32)
    S = (q @ k.T).astype(_F32)
    x = (S.astype(np.float64) * np.float64(_SCALE_LOG2) - lse2[:, None].astype(np.float64)).astype(_F32)
    P = np.exp2(x.astype(np.float64)).astype(_F32)
    P[np.triu(np.ones((T, T), bool), 1)] = 0
    dP = (do @ v.T).astype(_F32)
    dS = (P * (dP - delta[:, None]).astype(_F32)).astype(_F32)
    dSb = _bf16(dS)
    dv = _bf16((_bf16(P).T @ do).astype(_F32))
    dk = _bf16((dSb.T @ q).astype(_F32) * _SCALE)
    dq = _bf16((dSb @ k).astype(_F32) * _SCALE)
    return dq, dk, dv

