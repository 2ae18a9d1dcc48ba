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
