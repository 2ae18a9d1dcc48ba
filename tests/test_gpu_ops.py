"""Per-kernel parity on the GPU, through the C ABI (include/nc_ops.h), against
the fp64 oracle's component functions on the same seeded inputs.

Matrix products are checked bit-exactly on small-integer inputs (every
product and every fp32 partial sum is then exact, so any layout, tiling or
reduction-order bug shows up as a wrong integer).  bf16 outputs are compared
with the round-to-nearest-even of the exact result.  Floating-point
components use the fp32-mode bar (max relative error <= 1e-5 for fp32
storage) or a bound derived from bf16 output rounding (2^-8 relative per
element -> max relative error <= 1e-2, cosine >= 0.9999)."""
import math

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
import synthdata
from _util import dev, host, empty, zeros, max_rel_err, cosine
from _util import attention_fwd_rounding_model, attention_bwd_rounding_model

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import decoder_only_transformer_d20_amd as nc  # noqa: E402

DT = {"f32": 0, "bf16": 1}


def _ints(rng, shape, lo=-3, hi=3):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def _sync():
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# matrix products
# ---------------------------------------------------------------------------
MM_CASES = [
    # dtype, portable, M, N, K  (several tiles of every kernel + ragged tails)
    ("f32", 1, 320, 192, 384),
    ("bf16", 1, 320, 192, 384),
    ("bf16", 0, 384, 640, 320),      # 128 x 128 tiles
    ("bf16", 0, 768, 1280, 640),     # 256 x 256 tiles
    ("bf16", 0, 512, 384, 2048),     # 256 x 128 tiles
    # M, N odd multiples of 128 (>= 1024): 256 x 256 tiles whose last row /
    # column of tiles is shifted back by 128 (bf16 k-major stores and the
    # transposed-operand fp32 products); the other layouts take 128 x 128
    ("bf16", 0, 1152, 1408, 320),
    ("bf16", 0, 1152, 1280, 192),
    ("bf16", 0, 2048, 1920, 128),
]


@pytest.mark.parametrize("dtype,portable,M,N,K", MM_CASES)
@pytest.mark.parametrize("pt,qt", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_matmul_exact_integers(dtype, portable, M, N, K, pt, qt):
    rng = np.random.default_rng(100 + M + 7 * pt + 3 * qt)
    P = _ints(rng, (M, K))
    Q = _ints(rng, (N, K))
    want = P.astype(np.int64) @ Q.astype(np.int64).T
    Pd = dev(P.T.copy() if pt else P, dtype)
    Qd = dev(Q.T.copy() if qt else Q, dtype)
    C = empty((M, N), "f32")
    nc.ops.matmul(DT[dtype], pt, qt, M, N, K, Pd, Qd, C, 1, 1, None, portable, None)
    _sync()
    np.testing.assert_array_equal(host(C), want)
    # stored in the operand dtype: the RNE rounding of the exact result
    Cs = empty((M, N), dtype)
    nc.ops.matmul(DT[dtype], pt, qt, M, N, K, Pd, Qd, Cs, 0, 1, None, portable, None)
    _sync()
    wantr = want.astype(np.float32)
    if dtype == "bf16":
        wantr = synthdata.round_to_bf16(wantr)
    np.testing.assert_array_equal(host(Cs, dtype), wantr)


@pytest.mark.parametrize("K,S", [(4096, 4), (4096, 5), (832, 7)])
@pytest.mark.parametrize("dtype,portable", [("f32", 1), ("bf16", 1), ("bf16", 0)])
def test_matmul_split_k_exact(dtype, portable, K, S):
    """Split-K with even and uneven splits (split i takes the 64-wide k
    blocks [i nb/S, (i+1) nb/S)), exact on integer data."""
    rng = np.random.default_rng(7)
    M, N = 256, 384
    P = _ints(rng, (K, M))     # stored [K][M]: the weight-gradient layout
    Q = _ints(rng, (K, N))
    want = P.astype(np.int64).T @ Q.astype(np.int64)
    C = empty((M, N), "f32")
    part = empty((S * M * N,), "f32")
    nc.ops.matmul(DT[dtype], 1, 1, M, N, K, dev(P, dtype), dev(Q, dtype), C, 1, S, part, portable, None)
    _sync()
    np.testing.assert_array_equal(host(C), want)


@pytest.mark.parametrize("M,N,S", [(1152, 1920, 3), (1920, 1280, 1), (1920, 1920, 5)])
def test_matmul_split_k_shifted_tiles_exact(M, N, S):
    """Weight-gradient products whose output sides are odd multiples of 128
    (the d30 widths): the last tiles overlap their neighbours; every output
    must be written once, exactly, with and without split-K."""
    rng = np.random.default_rng(11 + S)
    K = 1024
    P = _ints(rng, (K, M))
    Q = _ints(rng, (K, N))
    want = P.astype(np.int64).T @ Q.astype(np.int64)
    C = zeros((M, N), "f32")
    part = empty((S * M * N,), "f32")
    nc.ops.matmul(1, 1, 1, M, N, K, dev(P, "bf16"), dev(Q, "bf16"), C, 1, S, part, 0, None)
    _sync()
    np.testing.assert_array_equal(host(C), want)


@pytest.mark.parametrize("dtype,portable", [("f32", 1), ("bf16", 1), ("bf16", 0)])
@pytest.mark.parametrize("qt,batch,M,N,K", [(0, 3, 256, 256, 384), (1, 5, 128, 384, 256), (0, 80, 256, 256, 256),
                                             (1, 2, 512, 1280, 256)])
def test_matmul_batched_axpby_exact(dtype, portable, qt, batch, M, N, K):
    """Batched products (items at uneven strides) with and without the
    alpha acc + gamma aux epilogue, exact on small integers with alpha,
    gamma powers of two: every product, sum and scaling is exact, so the
    stored result is the rounding of the exact value."""
    rng = np.random.default_rng(200 + batch + qt)
    pad = 64                                          # items not packed back to back
    P = _ints(rng, (batch, M * K + pad))
    Q = _ints(rng, (batch, N * K + pad))
    A = _ints(rng, (batch, M * N + pad))
    Pd, Qd, Ad = dev(P, dtype), dev(Q, dtype), dev(A, dtype)
    for alpha, gamma, with_aux in ((1.0, 0.0, False), (2.0, -0.5, True), (-4.0, 0.25, True)):
        C = empty((batch, M * N + pad), dtype)
        nc.ops.matmul_batched(DT[dtype], qt, batch, M, N, K, Pd, M * K + pad, Qd, N * K + pad, C, M * N + pad,
                              Ad if with_aux else None, M * N + pad, alpha, gamma, 0, portable, None)
        _sync()
        got = host(C, dtype)
        for b in range(batch):
            Pb = P[b, :M * K].reshape(M, K).astype(np.int64)
            Qb = Q[b, :N * K].astype(np.int64)
            Qb = Qb.reshape(K, N).T if qt else Qb.reshape(N, K)
            want = (Pb @ Qb.T).astype(np.float64)
            if with_aux:
                want = alpha * want + gamma * A[b, :M * N].reshape(M, N)
            want = want.astype(np.float32)
            if dtype == "bf16":
                want = synthdata.round_to_bf16(want)
            np.testing.assert_array_equal(got[b, :M * N].reshape(M, N), want, err_msg=f"item {b}")


@pytest.mark.parametrize("portable", [0, 1])
@pytest.mark.parametrize("batch,n,K", [(3, 1280, 512), (5, 640, 256), (2, 384, 1280), (80, 256, 128)])
def test_matmul_batched_symmetric_exact(portable, batch, n, K):
    """sym = 1, the Newton-Schulz products: A_b = X_b X_b^T and then
    B_b = 2 A_b A_b - 0.5 A_b, bit for bit against numpy; the matrix-core
    kernel computes the upper tiles (256 x 256 for n = 1280, 128 x 128 for
    640 and 384) and mirrors the rest.  X is sparse in {-1, 0, 1} (6 %
    nonzero), so every entry of A is an integer of magnitude < 256 (exact
    in bf16) and every partial sum of A A stays below 2^24 (exact in
    fp32): each result is the rounding of the exact value."""
    rng = np.random.default_rng(300 + n + batch)
    X = rng.choice(np.array([-1.0, 0.0, 1.0], np.float32), size=(batch, n * K), p=[0.03, 0.94, 0.03])
    Xd = dev(X, "bf16")
    A = empty((batch, n * n), "bf16")
    nc.ops.matmul_batched(1, 0, batch, n, n, K, Xd, n * K, Xd, n * K, A, n * n, None, 0, 1.0, 0.0, 1, portable, None)
    B = empty((batch, n * n), "bf16")
    nc.ops.matmul_batched(1, 0, batch, n, n, n, A, n * n, A, n * n, B, n * n, A, n * n, 2.0, -0.5, 1, portable, None)
    _sync()
    ga, gb = host(A, "bf16"), host(B, "bf16")
    for b in range(batch):
        Xb = X[b].reshape(n, K).astype(np.int64)
        Ab = Xb @ Xb.T
        assert np.abs(Ab).max() < 256 and (np.abs(Ab) @ np.abs(Ab)).max() * 2 < 2 ** 24
        np.testing.assert_array_equal(ga[b].reshape(n, n), synthdata.round_to_bf16(Ab.astype(np.float32)),
                                      err_msg=f"A item {b}")
        Ar = ga[b].reshape(n, n).astype(np.float64)         # the rounded A the second product reads
        want = synthdata.round_to_bf16((2.0 * (Ar @ Ar) - 0.5 * Ar).astype(np.float32))
        np.testing.assert_array_equal(gb[b].reshape(n, n), want, err_msg=f"B item {b}")


def test_matmul_batched_rejects():
    P = dev(np.zeros(2 * 192 * 128, np.float32), "bf16")
    C = empty((2 * 192 * 192,), "bf16")
    cases = (((1, 0, 2, 192, 192, 128, P, 192 * 128, P, 192 * 128, C, 192 * 192, None, 0, 1.0, 0.0, 0, 0), -6),
             ((1, 0, 2, 128, 128, 128, P, 128 * 128 + 4, P, 0, C, 0, None, 0, 1.0, 0.0, 0, 1), -1),
             ((1, 2, 2, 128, 128, 128, P, 0, P, 0, C, 0, None, 0, 1.0, 0.0, 0, 1), -1),
             ((1, 0, 0, 128, 128, 128, P, 0, P, 0, C, 0, None, 0, 1.0, 0.0, 0, 1), -1),
             ((1, 0, 2, 128, 100, 128, P, 0, P, 0, C, 0, None, 0, 1.0, 0.0, 0, 1), -2),
             ((1, 0, 2, 128, 256, 128, P, 0, P, 0, C, 0, None, 0, 1.0, 0.0, 1, 0), -2),
             ((1, 0, 2, 128, 128, 128, P, 0, P, 0, C, 0, None, 0, 1.0, 0.0, 2, 0), -1))
    for args, status in cases:
        with pytest.raises(nc.NcError) as e:
            nc.ops.matmul_batched(*args, None)
        assert e.value.status == status, (args[1:6], e.value.status)


def test_matmul_full_size_sampled_rows():
    """The d20 QKV product at its real shape (65,536 x 3,840 x 1,280), checked
    exactly on sampled rows."""
    rng = np.random.default_rng(8)
    M, N, K = 65536, 3840, 1280
    P = _ints(rng, (M, K), -2, 2)
    Q = _ints(rng, (N, K), -2, 2)
    C = empty((M, N), "f32")
    nc.ops.matmul(1, 0, 0, M, N, K, dev(P, "bf16"), dev(Q, "bf16"), C, 1, 1, None, 0, None)
    _sync()
    rows = np.concatenate([[0, M - 1], rng.choice(M, 30, replace=False)])
    got = host(C[torch.from_numpy(rows).cuda()])
    np.testing.assert_array_equal(got, P[rows].astype(np.int64) @ Q.astype(np.int64).T)


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,rows,d", [("f32", 130, 128), ("bf16", 300, 1280), ("bf16", 68, 1920)])
def test_rmsnorm_fwd_bwd(dtype, rows, d):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((rows, d)).astype(np.float32) * 2.5
    dy = rng.standard_normal((rows, d)).astype(np.float32)
    res = rng.standard_normal((rows, d)).astype(np.float32)
    if dtype == "bf16":
        x, dy, res = (synthdata.round_to_bf16(a) for a in (x, dy, res))
    eps = 1e-6
    y_want, r_want = oracle.rmsnorm(x.astype(np.float64), eps)
    xd, yd, rd = dev(x, dtype), empty((rows, d), dtype), empty((rows,), "f32")
    nc.ops.rmsnorm_fwd(DT[dtype], rows, d, eps, xd, yd, rd, None)
    _sync()
    tol = 1e-5 if dtype == "f32" else 1e-2
    assert max_rel_err(host(rd), r_want) <= 1e-6
    assert max_rel_err(host(yd, dtype), y_want) <= tol
    # backward from the kernel's own stored y and r, with and without residual
    y_used = host(yd, dtype)
    dx_want = oracle.rmsnorm_bwd(y_used, host(rd), dy.astype(np.float64))
    for acc in (0, 1):
        io = dev(res, dtype)
        nc.ops.rmsnorm_bwd(DT[dtype], rows, d, yd, rd, dev(dy, dtype), io, acc, None)
        _sync()
        want = dx_want + (res if acc else 0)
        assert max_rel_err(host(io, dtype), want) <= tol
        assert cosine(host(io, dtype), want) >= 0.9999


# ---------------------------------------------------------------------------
# rotary table
# ---------------------------------------------------------------------------
def test_rope_table_matches_fp64_angles():
    T, Q = 2048, 128
    tab = empty((T, Q // 2, 2), "f32")
    nc.ops.rope_table(T, Q, 10000.0, tab, None)
    _sync()
    phi = oracle.rope_angles(T, Q, 10000.0)
    got = host(tab)
    assert np.max(np.abs(got[..., 0] - np.cos(phi))) <= 1e-7
    assert np.max(np.abs(got[..., 1] - np.sin(phi))) <= 1e-7


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
ATT_CASES = [
    # dtype, portable, B, T, H, Q
    ("f32", 1, 2, 128, 2, 64),
    ("bf16", 1, 2, 192, 2, 128),
    ("bf16", 0, 2, 256, 2, 128),
    ("bf16", 0, 1, 640, 3, 128),
    ("bf16", 0, 1, 2048, 10, 128),   # one row of the d20 launch: every head, full row length
    ("bf16", 0, 2, 192, 2, 128),     # T % 128 == 64: half-empty last query and key blocks
    ("bf16", 0, 1, 320, 3, 128),
    ("bf16", 0, 1, 448, 2, 128),     # 256-query blocks, a 128-query block and a 64-query block
    ("bf16", 0, 1, 64, 2, 128),      # the 64-query block alone
]


def _qkv(rng, B, T, H, Q, dtype):
    a = rng.standard_normal((B, T, 3, H, Q)).astype(np.float32)
    return synthdata.round_to_bf16(a) if dtype == "bf16" else a


@pytest.mark.parametrize("dtype,portable,B,T,H,Q", ATT_CASES)
def test_attention_fwd(dtype, portable, B, T, H, Q):
    rng = np.random.default_rng(10 + T)
    qkv = _qkv(rng, B, T, H, Q, dtype)
    o = empty((B, T, H, Q), dtype)
    lse = empty((B, H, T), "f32")
    nc.ops.attention_fwd(DT[dtype], B, T, H, Q, dev(qkv, dtype), o, lse, portable, None)
    _sync()
    og, lg = host(o, dtype), host(lse)
    tol = 1e-5 if dtype == "f32" else 1e-2
    for b in range(B):
        q, k, v = (qkv[b, :, i].astype(np.float64) for i in range(3))
        want = oracle.causal_attention(q, k, v)
        assert max_rel_err(og[b], want) <= tol
        assert cosine(og[b], want) >= 0.99995
        for h in range(H):
            S = q[:, h] @ k[:, h].T / math.sqrt(Q)
            S[np.triu(np.ones((T, T), bool), 1)] = -np.inf
            np.testing.assert_allclose(lg[b, h], logsumexp(S, axis=1), rtol=1e-5, atol=1e-5)


# every case with the recompute path; the bf16 matrix-core cases also with
# the stored-dS path (nc_op_attention_bwd_ds)
ATT_BWD_CASES = [c + (0,) for c in ATT_CASES] + [c + (1,) for c in ATT_CASES if c[0] == "bf16" and c[1] == 0]


@pytest.mark.parametrize("dtype,portable,B,T,H,Q,stored_ds", ATT_BWD_CASES)
@pytest.mark.parametrize("with_rope", [0, 1])
def test_attention_bwd(dtype, portable, B, T, H, Q, stored_ds, with_rope):
    """dq, dk, dv against the oracle; stored_ds = 1 takes the path that
    writes dS^T to a scratch buffer and forms dQ from it.  The scratch is
    filled with NaN first: a piece the dQ kernel read but the dK/dV kernel
    never wrote would show."""
    rng = np.random.default_rng(20 + T)
    qkv = _qkv(rng, B, T, H, Q, dtype)
    dout = rng.standard_normal((B, T, H, Q)).astype(np.float32)
    if dtype == "bf16":
        dout = synthdata.round_to_bf16(dout)
    qkvd = dev(qkv, dtype)
    o = empty((B, T, H, Q), dtype)
    lse = empty((B, H, T), "f32")
    nc.ops.attention_fwd(DT[dtype], B, T, H, Q, qkvd, o, lse, portable, None)
    tab = empty((T, Q // 2, 2), "f32")
    nc.ops.rope_table(T, Q, 10000.0, tab, None)
    delta = empty((B, H, T), "f32")
    dqkv = zeros((B, T, 3, H, Q), dtype)
    if stored_ds:
        nbytes = nc.ops.attention_ds_bytes(B, T, H)
        nq = (T + 127) // 128
        assert nbytes == B * H * nq * (nq + 1) * 64 * 128 * 2
        ds = torch.full((nbytes // 2,), float("nan"), dtype=torch.bfloat16, device="cuda")
        nc.ops.attention_bwd_ds(B, T, H, Q, qkvd, o, dev(dout, dtype), lse, delta, dqkv,
                                tab if with_rope else None, ds, None)
    else:
        nc.ops.attention_bwd(DT[dtype], B, T, H, Q, qkvd, o, dev(dout, dtype), lse, delta, dqkv,
                             tab if with_rope else None, portable, None)
    _sync()
    got = host(dqkv, dtype)
    phi = oracle.rope_angles(T, Q, 10000.0)
    tol = 1e-4 if dtype == "f32" else 2e-2
    for b in range(B):
        q, k, v = (qkv[b, :, i].astype(np.float64) for i in range(3))
        dq, dk, dv = oracle.causal_attention_bwd(q, k, v, dout[b].astype(np.float64))
        if with_rope:
            dq, dk = oracle.rope(dq, phi, inverse=True), oracle.rope(dk, phi, inverse=True)
        for i, want in enumerate((dq, dk, dv)):
            assert max_rel_err(got[b, :, i], want) <= tol, ("dq", "dk", "dv")[i]
            assert cosine(got[b, :, i], want) >= 0.9999, ("dq", "dk", "dv")[i]


@pytest.mark.parametrize("T,H", [(448, 2), (2048, 2)])
def test_attention_matches_rounding_model(T, H):
    """The matrix-core forward and backward against a step-by-step model of
    their own arithmetic (_util.attention_*_rounding_model: every rounding
    the kernels make, in fp32 and bf16).  What the model leaves out -- the
    order of the fp32 sums and the hardware exp2 / log2 / reciprocal, a few
    fp32 ulps each -- moves a value across a bf16 rounding boundary about
    once in 2^13 roundings.  A flip moves one rounded value by one bf16
    ulp of itself: an output by one ulp, a P or dS term by one ulp of the
    term, which in a sum of terms (dq, dk, dv) is at most an ulp of the
    sum's scale even where the sum itself cancels to a small value.  So
    the bar is: at least 99 % of the bf16 outputs bitwise equal to the
    model's, every difference within one bf16 ulp of the tensor's largest
    magnitude, and the log-sum-exp within 1e-6.  T = 448 runs the full, the
    128-row and the 64-row query blocks; T = 2048 the d20 row length."""
    rng = np.random.default_rng(40 + T)
    B, Q = 1, 128
    qkv = _qkv(rng, B, T, H, Q, "bf16")
    dout = synthdata.round_to_bf16(rng.standard_normal((B, T, H, Q)).astype(np.float32))
    qkvd = dev(qkv, "bf16")
    o = empty((B, T, H, Q), "bf16")
    lse = empty((B, H, T), "f32")
    nc.ops.attention_fwd(DT["bf16"], B, T, H, Q, qkvd, o, lse, 0, None)
    delta = empty((B, H, T), "f32")
    dqkv = zeros((B, T, 3, H, Q), "bf16")
    nc.ops.attention_bwd(DT["bf16"], B, T, H, Q, qkvd, o, dev(dout, "bf16"), lse, delta, dqkv, None, 0, None)
    _sync()
    og, lg, gg = host(o, "bf16"), host(lse), host(dqkv, "bf16")
    for h in range(H):
        q, k, v = (qkv[0, :, i, h].astype(np.float64) for i in range(3))
        mo, ml = attention_fwd_rounding_model(q, k, v)
        np.testing.assert_allclose(lg[0, h], ml, rtol=1e-6, atol=1e-6)
        grads = attention_bwd_rounding_model(q, k, v, mo, ml, dout[0, :, h].astype(np.float64))
        for name, got, want in [("o", og[0, :, h], mo)] + [(n, gg[0, :, i, h], w) for i, (n, w) in
                                                          enumerate(zip(("dq", "dk", "dv"), grads))]:
            same = float(np.mean(got == want))
            top = np.max(np.abs(want))
            ulps = np.max(np.abs(got - want)) / 2.0 ** (np.floor(np.log2(top)) - 7)
            print(f"T={T} h={h} {name}: bitwise equal {same:.5f}, largest difference {ulps:.3f} ulp of the "
                  f"largest magnitude", flush=True)
            assert same >= 0.99, name
            assert ulps <= 1.0, name


# ---------------------------------------------------------------------------
# embedding
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,d,V,n", [("f32", 128, 512, 1000), ("bf16", 1280, 512, 1000),
                                         ("bf16", 192, 65536, 5000), ("f32", 64, 300, 1),
                                         ("bf16", 1280, 65536, 65536)])   # the d20 launch: id 0 ~9k times
def test_embedding_gather_bitwise_and_gradient(dtype, d, V, n):
    """Gather is a bitwise row copy (an id outside [0, V) gives a NaN row);
    the gradient (a per-id sum of rows) is checked against an fp64
    np.add.at, with and without accumulation, with ids outside [0, V)
    dropped, and is bitwise identical across calls."""
    rng = np.random.default_rng(30)
    E = rng.standard_normal((V, d)).astype(np.float32)
    if dtype == "bf16":
        E = synthdata.round_to_bf16(E)
    cfg = synthdata.get_config("d20")
    idx = (synthdata.make_tokens(cfg.with_(batch=1, seq_len=max(n, 2)), rows=1)[0].ravel()[:n] % V).astype(np.int32)
    x = empty((n, d), dtype)
    nc.ops.embed_fwd(DT[dtype], n, d, V, dev(E, dtype), dev(idx), x, None)
    _sync()
    np.testing.assert_array_equal(host(x, dtype), E[idx])
    if n > 4:
        oob = idx.copy()
        oob[2], oob[4] = V, -1
        nc.ops.embed_fwd(DT[dtype], n, d, V, dev(E, dtype), dev(oob), x, None)
        _sync()
        xo = host(x, dtype)
        assert np.all(np.isnan(xo[[2, 4]]))
        keep = np.setdiff1d(np.arange(n), [2, 4])
        np.testing.assert_array_equal(xo[keep], E[oob[keep]])
    g = rng.standard_normal((n, d)).astype(np.float32)
    if dtype == "bf16":
        g = synthdata.round_to_bf16(g)
    bad = idx.copy()
    if n > 4:
        bad[1], bad[3] = -5, V + 7                 # dropped
    scratch = empty((nc.ops.embed_bwd_scratch_bytes(n, d) // 4 + 1,), "f32")
    G, I = dev(g, dtype), dev(bad)
    dE = zeros((V, d), "f32")
    nc.ops.embed_bwd(DT[dtype], n, d, V, G, I, dE, 0, scratch, None)
    _sync()
    keep = (bad >= 0) & (bad < V)
    want = np.zeros((V, d))
    np.add.at(want, bad[keep], g[keep].astype(np.float64))
    got = host(dE)
    assert max_rel_err(got, want) <= 1e-6
    assert np.all(got[np.setdiff1d(np.arange(V), bad[keep])] == 0)
    # bitwise repeatable; accumulate adds onto what is there
    dE2 = dev(np.full((V, d), 7.0, np.float32))
    nc.ops.embed_bwd(DT[dtype], n, d, V, G, I, dE2, 0, scratch, None)
    nc.ops.embed_bwd(DT[dtype], n, d, V, G, I, dE, 1, scratch, None)
    _sync()
    np.testing.assert_array_equal(host(dE2), got)
    assert max_rel_err(host(dE), 2 * want) <= 1e-6


# ---------------------------------------------------------------------------
# fused unembedding + cross-entropy
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,portable,n,d,V", [("f32", 1, 128, 128, 512), ("bf16", 1, 256, 256, 640),
                                                  ("bf16", 0, 256, 256, 640), ("bf16", 0, 512, 1280, 4096)])
def test_head_ce_forward(dtype, portable, n, d, V):
    rng = np.random.default_rng(40)
    xf = rng.standard_normal((n, d)).astype(np.float32)
    U = (rng.standard_normal((V, d)) / math.sqrt(d)).astype(np.float32) * 3
    if dtype == "bf16":
        xf, U = synthdata.round_to_bf16(xf), synthdata.round_to_bf16(U)
    tgt = rng.integers(0, V, size=n).astype(np.int32)
    tgt[5] = -1
    tgt[7] = V - 1
    tgt[9] = 0
    ce, lse = empty((n,), "f32"), empty((n,), "f32")
    scratch = empty((nc.ops.head_scratch_bytes(DT[dtype], n, d, V, portable) // 4 + 1,), "f32")
    nc.ops.head_ce_fwd(DT[dtype], n, d, V, dev(xf, dtype), dev(U, dtype), dev(tgt), ce, lse, scratch, portable, None)
    _sync()
    z = xf.astype(np.float64) @ U.astype(np.float64).T
    want = oracle.cross_entropy(z, tgt)
    np.testing.assert_allclose(host(ce), want, rtol=1e-5, atol=2e-5)
    np.testing.assert_allclose(host(lse), logsumexp(z, axis=1), rtol=1e-5, atol=2e-5)
    assert host(ce)[5] == 0.0


def test_mfma_loop_probe_runs_every_iteration():
    """The throughput probe behind bench.py's measured MFMA peak: each
    thread's sink value is a sum of `iters` identical iterations of products,
    so doubling iters doubles it (to fp32 rounding), and it is finite and
    non-zero."""
    blocks = 8
    s1, s2 = empty((blocks * 256,), "f32"), empty((blocks * 256,), "f32")
    nc.ops.mfma_loop(100, blocks, s1, None)
    nc.ops.mfma_loop(200, blocks, s2, None)
    torch.cuda.synchronize()
    a, b = host(s1), host(s2)
    assert np.all(np.isfinite(a)) and np.all(a > 0)
    np.testing.assert_allclose(b, 2 * a, rtol=1e-5)
