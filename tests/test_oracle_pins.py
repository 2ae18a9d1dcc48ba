"""Pins for the fp64 oracle: each check compares it with something other than
itself -- a closed form, an invariant, a special case that reduces to a
textbook routine, brute force on tiny inputs, or fp64 finite differences --
chosen so that a dropped term, a wrong sign or index, or a transposed operand
anywhere in the oracle fails at least one of them."""
import cmath
import math

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
import synthdata
from synthdata import Config

MICRO = Config("micro", 2, 16, 2, 8, 64, 32, 2, 8, "f32", 11)


def _rng(seed=0):
    return np.random.default_rng(seed)


def _micro_params(cfg=MICRO, seed=5, scale=1.0):
    rng = _rng(seed)
    flat = np.zeros(synthdata.param_count(cfg))
    for name, layer, r, c, off in synthdata.param_layout(cfg):
        std = 1.0 if name == "E" else scale / math.sqrt(c)
        flat[off:off + r * c] = rng.standard_normal(r * c) * std
    return flat, synthdata.split_params(cfg, flat)


# --------------------------------------------------------------------------
# RMSNorm
# --------------------------------------------------------------------------
def test_rmsnorm_unit_rms_and_scale_invariance():
    x = _rng(1).standard_normal((7, 33)) * 3.0
    y, r = oracle.rmsnorm(x, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-14)
    y2, _ = oracle.rmsnorm(x * 17.5, 0.0)
    np.testing.assert_allclose(y2, y, rtol=1e-13, atol=1e-14)
    # r is the reciprocal RMS: the norm of a row of x is sqrt(d)/r
    np.testing.assert_allclose(np.linalg.norm(x, axis=1), math.sqrt(33) / r, rtol=1e-13)


def test_rmsnorm_eps_enters_under_the_root():
    x = np.array([[3.0, 4.0]])           # mean square 12.5
    y, r = oracle.rmsnorm(x, 0.5)
    assert r[0] == pytest.approx(1.0 / math.sqrt(13.0), rel=1e-15)


def test_rmsnorm_bwd_orthogonal_to_input_and_fd():
    rng = _rng(2)
    x = rng.standard_normal((5, 12))
    y, r = oracle.rmsnorm(x, 0.0)
    dy = rng.standard_normal(x.shape)
    dx = oracle.rmsnorm_bwd(y, r, dy)
    # scale invariance of y => <dx, x> = 0 row by row
    np.testing.assert_allclose(np.sum(dx * x, axis=1), 0.0, atol=1e-12)
    for eps in (0.0, 1e-2):
        y, r = oracle.rmsnorm(x, eps)
        dx = oracle.rmsnorm_bwd(y, r, dy)
        v = rng.standard_normal(x.shape)
        h = 1e-6
        fd = (np.sum(oracle.rmsnorm(x + h * v, eps)[0] * dy)
              - np.sum(oracle.rmsnorm(x - h * v, eps)[0] * dy)) / (2 * h)
        assert fd == pytest.approx(np.sum(dx * v), rel=1e-7)


# --------------------------------------------------------------------------
# rotary positions
# --------------------------------------------------------------------------
def test_rope_matches_complex_rotation_brute_force():
    T, H, Q, base = 5, 2, 8, 10000.0
    x = _rng(3).standard_normal((T, H, Q))
    y = oracle.rope(x, oracle.rope_angles(T, Q, base))
    for t in range(T):
        for h in range(H):
            for i in range(Q // 2):
                z = complex(x[t, h, 2 * i], x[t, h, 2 * i + 1])
                w = z * cmath.exp(1j * t * base ** (-2.0 * i / Q))
                assert y[t, h, 2 * i] == pytest.approx(w.real, abs=1e-13)
                assert y[t, h, 2 * i + 1] == pytest.approx(w.imag, abs=1e-13)


def test_rope_invariants():
    T, H, Q = 9, 3, 16
    rng = _rng(4)
    phi = oracle.rope_angles(T, Q, 10000.0)
    x = rng.standard_normal((T, H, Q))
    y = oracle.rope(x, phi)
    # t = 0 is the identity; pair norms are preserved; inverse undoes it
    np.testing.assert_array_equal(y[0], x[0])
    np.testing.assert_allclose(y[..., 0::2] ** 2 + y[..., 1::2] ** 2,
                               x[..., 0::2] ** 2 + x[..., 1::2] ** 2, rtol=1e-12)
    np.testing.assert_allclose(oracle.rope(y, phi, inverse=True), x, atol=1e-13)
    # the inverse is the transpose: <R x, g> = <x, R^T g>
    g = rng.standard_normal(x.shape)
    assert np.sum(y * g) == pytest.approx(np.sum(x * oracle.rope(g, phi, inverse=True)), rel=1e-12)
    # relative position: <R_m q, R_n k> depends only on m - n
    q = rng.standard_normal(Q)
    k = rng.standard_normal(Q)
    Qs = np.broadcast_to(q, (T, 1, Q)).copy()
    Ks = np.broadcast_to(k, (T, 1, Q)).copy()
    rq, rk = oracle.rope(Qs, phi)[:, 0], oracle.rope(Ks, phi)[:, 0]
    for delta in (0, 1, 3):
        dots = [rq[m] @ rk[m - delta] for m in range(delta, T)]
        np.testing.assert_allclose(dots, dots[0], rtol=1e-11)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------
def _attention_brute_force(q, k, v):
    T, H, Q = q.shape
    o = np.zeros_like(q)
    for h in range(H):
        for t in range(T):
            s = [sum(q[t, h, e] * k[j, h, e] for e in range(Q)) / math.sqrt(Q) for j in range(t + 1)]
            mx = max(s)
            w = [math.exp(si - mx) for si in s]
            tot = sum(w)
            for j in range(t + 1):
                o[t, h] += (w[j] / tot) * v[j, h]
    return o


def test_attention_brute_force_tiny():
    rng = _rng(5)
    q, k, v = (rng.standard_normal((6, 2, 4)) for _ in range(3))
    np.testing.assert_allclose(oracle.causal_attention(q, k, v),
                               _attention_brute_force(q, k, v), rtol=1e-12, atol=1e-13)


def test_attention_closed_forms():
    rng = _rng(6)
    T, H, Q = 10, 2, 8
    q, k, v = (rng.standard_normal((T, H, Q)) for _ in range(3))
    # T = 1: the only key is the query's own -> o = v
    np.testing.assert_allclose(oracle.causal_attention(q[:1], k[:1], v[:1]), v[:1], rtol=1e-14)
    # q = 0: uniform weights over the causal prefix -> prefix mean of v
    o = oracle.causal_attention(np.zeros_like(q), k, v)
    prefix_mean = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None, None]
    np.testing.assert_allclose(o, prefix_mean, rtol=1e-12, atol=1e-14)
    # softmax rows sum to one: v = 1 gives o = 1
    np.testing.assert_allclose(oracle.causal_attention(q, k, np.ones_like(v)), 1.0, rtol=1e-14)


def test_attention_causality_bitwise():
    rng = _rng(7)
    T, H, Q, t = 12, 2, 8, 6
    q, k, v = (rng.standard_normal((T, H, Q)) for _ in range(3))
    o = oracle.causal_attention(q, k, v)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[t + 1:] += 5.0
    k2[t + 1:] -= 3.0
    v2[t + 1:] *= -7.0
    o2 = oracle.causal_attention(q2, k2, v2)
    np.testing.assert_array_equal(o2[:t + 1], o[:t + 1])


def test_attention_bwd_finite_differences():
    rng = _rng(8)
    T, H, Q = 7, 2, 4
    q, k, v = (rng.standard_normal((T, H, Q)) for _ in range(3))
    do = rng.standard_normal((T, H, Q))
    dq, dk, dv = oracle.causal_attention_bwd(q, k, v, do)
    h = 1e-6
    for grad, which in ((dq, 0), (dk, 1), (dv, 2)):
        dirn = rng.standard_normal((T, H, Q))
        args_p = [q, k, v]
        args_m = [q, k, v]
        args_p = [a + h * dirn if i == which else a for i, a in enumerate(args_p)]
        args_m = [a - h * dirn if i == which else a for i, a in enumerate(args_m)]
        fd = (np.sum(oracle.causal_attention(*args_p) * do)
              - np.sum(oracle.causal_attention(*args_m) * do)) / (2 * h)
        assert fd == pytest.approx(np.sum(grad * dirn), rel=1e-7)


# --------------------------------------------------------------------------
# squared ReLU, cross-entropy, bits per byte
# --------------------------------------------------------------------------
def test_relu2_closed_form():
    h = np.array([-2.0, -0.0, 0.0, 0.5, 3.0])
    np.testing.assert_array_equal(oracle.model.relu2(h), [0.0, 0.0, 0.0, 0.25, 9.0])
    np.testing.assert_array_equal(oracle.model.relu2_grad(h), [0.0, 0.0, 0.0, 1.0, 6.0])


def test_cross_entropy_against_scipy_and_grad():
    rng = _rng(9)
    z = rng.standard_normal((6, 11)) * 4
    tgt = np.array([0, 10, 3, -1, 5, 5])
    ce = oracle.cross_entropy(z, tgt)
    for t in range(6):
        want = 0.0 if tgt[t] < 0 else logsumexp(z[t]) - z[t, tgt[t]]
        assert ce[t] == pytest.approx(want, rel=1e-14)
    dz = oracle.cross_entropy_grad(z, tgt, 0.25)
    np.testing.assert_allclose(dz.sum(axis=1), 0.0, atol=1e-15)
    np.testing.assert_array_equal(dz[3], 0.0)
    dirn = rng.standard_normal(z.shape)
    h = 1e-6
    fd = 0.25 * (oracle.cross_entropy(z + h * dirn, tgt).sum()
                 - oracle.cross_entropy(z - h * dirn, tgt).sum()) / (2 * h)
    assert fd == pytest.approx(np.sum(dz * dirn), rel=1e-7)


def test_uniform_logits_give_ln_v_and_bpb_closed_form():
    cfg = MICRO
    flat, p = _micro_params()
    p["U"][:] = 0.0
    idx, tgt = synthdata.make_tokens(cfg)
    tb = synthdata.make_token_bytes(cfg)
    out = oracle.train_step(cfg, p, idx, tgt, tb)
    V = cfg.vocab
    np.testing.assert_allclose(out["ce"], math.log(V), rtol=1e-14)
    assert out["loss"] == pytest.approx(math.log(V), rel=1e-14)
    n = tgt.size
    assert out["bpb"] == pytest.approx(math.log(V) / math.log(2) * n / tb[tgt].sum(), rel=1e-13)
    # the dz rows are (1/V - onehot)/N: the U gradient rows sum to zero over the vocab
    gU = out["grads"]["U"]
    np.testing.assert_allclose(gU.sum(axis=0), 0.0, atol=1e-13)


def test_loss_bpb_identity_and_ignored_targets():
    rng = _rng(10)
    ce = rng.random((3, 5)) * 4
    tgt = rng.integers(0, 20, size=(3, 5))
    tgt[1, 2] = -1
    tb = rng.integers(1, 9, size=20)
    loss, bpb = oracle.loss_bpb(ce, tgt, tb)
    valid = tgt >= 0
    assert loss == pytest.approx(ce[valid].sum() / valid.sum(), rel=1e-15)
    assert bpb == pytest.approx(loss * valid.sum() / (math.log(2) * tb[tgt[valid]].sum()), rel=1e-14)


# --------------------------------------------------------------------------
# whole model: special cases, causality, row independence, finite differences
# --------------------------------------------------------------------------
def _head_ce(cfg, x_final, U, tgt_row):
    ms = np.mean(x_final ** 2, axis=1)
    xf = x_final / np.sqrt(ms + cfg.rms_eps)[:, None]
    z = xf @ U.T
    return np.array([logsumexp(z[t]) - z[t, tgt_row[t]] for t in range(len(tgt_row))])


def _rms(x, eps):
    return x / np.sqrt(np.mean(x ** 2, axis=1) + eps)[:, None]


def test_model_zero_blocks_passes_embedding_through():
    cfg = MICRO
    _, p = _micro_params()
    for lp in p["layers"]:
        for k in lp:
            lp[k][:] = 0.0
    idx, tgt = synthdata.make_tokens(cfg)
    ce, _ = oracle.model_forward_row(p, idx[0], tgt[0], cfg)
    np.testing.assert_allclose(ce, _head_ce(cfg, p["E"][idx[0]], p["U"], tgt[0]), rtol=1e-12)


def test_model_uniform_attention_layer_closed_form():
    cfg = MICRO.with_(n_layer=1)
    _, p = _micro_params(cfg)
    lp = p["layers"][0]
    lp["Wq"][:] = 0.0
    lp["W1"][:] = 0.0          # MLP contributes relu(0)^2 W2 = 0
    idx, tgt = synthdata.make_tokens(cfg)
    x0 = p["E"][idx[0]]
    T = x0.shape[0]
    vv = _rms(x0, cfg.rms_eps) @ lp["Wv"].T
    ctx = np.cumsum(vv, axis=0) / np.arange(1, T + 1)[:, None]
    x1 = x0 + ctx @ lp["Wo"].T
    ce, _ = oracle.model_forward_row(p, idx[0], tgt[0], cfg)
    np.testing.assert_allclose(ce, _head_ce(cfg, x1, p["U"], tgt[0]), rtol=1e-11)


def test_model_mlp_only_layer_closed_form():
    cfg = MICRO.with_(n_layer=1)
    _, p = _micro_params(cfg)
    lp = p["layers"][0]
    lp["Wo"][:] = 0.0
    idx, tgt = synthdata.make_tokens(cfg)
    x0 = p["E"][idx[0]]
    hh = _rms(x0, cfg.rms_eps) @ lp["W1"].T
    x1 = x0 + (np.where(hh > 0, hh, 0.0) ** 2) @ lp["W2"].T
    ce, _ = oracle.model_forward_row(p, idx[0], tgt[0], cfg)
    np.testing.assert_allclose(ce, _head_ce(cfg, x1, p["U"], tgt[0]), rtol=1e-11)


def test_model_causality_bitwise():
    cfg = MICRO
    _, p = _micro_params()
    idx, tgt = synthdata.make_tokens(cfg)
    t = 3
    ce, _ = oracle.model_forward_row(p, idx[0], tgt[0], cfg)
    idx2 = idx[0].copy()
    idx2[t + 1:] = (idx2[t + 1:] + 7) % cfg.vocab
    ce2, _ = oracle.model_forward_row(p, idx2, tgt[0], cfg)
    np.testing.assert_array_equal(ce2[:t + 1], ce[:t + 1])
    assert not np.array_equal(ce2[t + 1:], ce[t + 1:])


def test_model_row_independence():
    cfg = MICRO
    _, p = _micro_params()
    idx, tgt = synthdata.make_tokens(cfg)
    tb = synthdata.make_token_bytes(cfg)
    full = oracle.train_step(cfg, p, idx, tgt, tb)
    r0 = oracle.train_step(cfg, p, idx, tgt, tb, rows=[0])
    r1 = oracle.train_step(cfg, p, idx, tgt, tb, rows=[1])
    np.testing.assert_allclose(full["ce"], r0["ce"] + r1["ce"], rtol=1e-15)
    for a, b, c in zip(_flat(full["grads"], cfg), _flat(r0["grads"], cfg), _flat(r1["grads"], cfg)):
        np.testing.assert_allclose(a, b + c, rtol=1e-12, atol=1e-16)


def test_ignored_targets_contribute_nothing():
    """A row whose targets are all ignored adds no loss and no gradient: the
    batch gradient equals the other row's part (same n_valid), exactly.  With
    no valid target anywhere the mean over the empty set is 0 and so is every
    gradient."""
    cfg = MICRO
    _, p = _micro_params()
    idx, tgt = synthdata.make_tokens(cfg)
    tb = synthdata.make_token_bytes(cfg)
    tgt = tgt.copy()
    tgt[1, :] = -1
    full = oracle.train_step(cfg, p, idx, tgt, tb)
    r0 = oracle.train_step(cfg, p, idx, tgt, tb, rows=[0])
    for a, b in zip(_flat(full["grads"], cfg), _flat(r0["grads"], cfg)):
        np.testing.assert_array_equal(a, b)
    assert full["loss"] == pytest.approx(full["ce"][0].sum() / tgt.shape[1], rel=1e-15)
    tgt[:] = -1
    none = oracle.train_step(cfg, p, idx, tgt, tb)
    assert none["loss"] == 0.0 and none["bpb"] == 0.0
    assert all(not np.any(g) for g in _flat(none["grads"], cfg))


def _flat(grads, cfg):
    out = []
    for name, layer, r, c, off in synthdata.param_layout(cfg):
        out.append((grads[name] if layer < 0 else grads["layers"][layer][name]).ravel())
    return out


def _loss_of(cfg, flat, idx, tgt, tb):
    return oracle.train_step(cfg, synthdata.split_params(cfg, flat), idx, tgt, tb,
                             want_grads=False)["loss"]


def test_model_gradient_finite_differences_every_tensor():
    cfg = MICRO
    flat, p = _micro_params()
    idx, tgt = synthdata.make_tokens(cfg)
    tgt = tgt.copy()
    tgt[1, 2] = -1                          # an ignored target too
    tb = synthdata.make_token_bytes(cfg)
    out = oracle.train_step(cfg, p, idx, tgt, tb)
    g = np.concatenate(_flat(out["grads"], cfg))
    rng = _rng(12)
    h = 1e-5
    for name, layer, r, c, off in synthdata.param_layout(cfg):
        n = r * c
        if name == "E":   # only rows that occur in idx have a gradient
            rows = np.unique(idx)
            picks = [off + int(rw) * c + int(rng.integers(c)) for rw in rows[:4]]
        else:
            picks = [off + int(j) for j in rng.choice(n, size=4, replace=False)]
        for j in picks:
            e = np.zeros_like(flat)
            e[j] = h
            fd = (_loss_of(cfg, flat + e, idx, tgt, tb) - _loss_of(cfg, flat - e, idx, tgt, tb)) / (2 * h)
            assert fd == pytest.approx(g[j], rel=1e-6, abs=1e-10), (name, layer, j)
    # one directional derivative over all parameters at once
    v = rng.standard_normal(flat.shape)
    fd = (_loss_of(cfg, flat + h * v, idx, tgt, tb) - _loss_of(cfg, flat - h * v, idx, tgt, tb)) / (2 * h)
    assert fd == pytest.approx(float(g @ v), rel=1e-7)


def test_block_step_gradient_finite_differences():
    cfg = MICRO.with_(n_layer=1, block_only=True, vocab=0)
    rng = _rng(13)
    flat, p = _micro_params(cfg)
    lp = p["layers"][0]
    x = rng.standard_normal((2, cfg.seq_len, cfg.d_model))
    dy = rng.standard_normal(x.shape)
    out = oracle.block_step(cfg, lp, x, dy)
    h = 1e-6
    # VJP w.r.t. x
    v = rng.standard_normal(x.shape)
    f = lambda xx: np.sum(oracle.block_step(cfg, lp, xx, dy)["y"] * dy)
    assert (f(x + h * v) - f(x - h * v)) / (2 * h) == pytest.approx(np.sum(out["dx"] * v), rel=1e-7)
    # VJP w.r.t. each weight
    for k in lp:
        w = rng.standard_normal(lp[k].shape)
        lpp = dict(lp); lpp[k] = lp[k] + h * w
        lpm = dict(lp); lpm[k] = lp[k] - h * w
        fd = (np.sum(oracle.block_step(cfg, lpp, x, dy)["y"] * dy)
              - np.sum(oracle.block_step(cfg, lpm, x, dy)["y"] * dy)) / (2 * h)
        assert fd == pytest.approx(np.sum(out["grads"][k] * w), rel=1e-7), k


# --------------------------------------------------------------------------
# token-weighted cross-entropy (the simplified GRPO's per-token advantages)
# --------------------------------------------------------------------------
def _weighted_objective(cfg, flat, idx, tgt, tb, w):
    out = oracle.train_step(cfg, synthdata.split_params(cfg, flat), idx, tgt, tb, want_grads=False)
    return oracle.weighted_loss(out["ce"], tgt, w)[1]


def test_weighted_gradient_finite_differences():
    """The weighted gradient is the derivative of sum_t w_t ce[t] / n_valid,
    by fp64 central differences along a random direction and on single
    entries, with weights of both signs and an ignored target."""
    cfg = MICRO
    flat, p = _micro_params(seed=21)
    idx, tgt = synthdata.make_tokens(cfg)
    tgt = tgt.copy()
    tgt[0, 3] = -1
    tb = synthdata.make_token_bytes(cfg)
    w = _rng(22).standard_normal(tgt.shape)
    g = np.concatenate(_flat(oracle.train_step(cfg, p, idx, tgt, tb, token_weights=w)["grads"], cfg))
    rng = _rng(23)
    h = 1e-5
    v = rng.standard_normal(flat.shape)
    fd = (_weighted_objective(cfg, flat + h * v, idx, tgt, tb, w)
          - _weighted_objective(cfg, flat - h * v, idx, tgt, tb, w)) / (2 * h)
    assert fd == pytest.approx(float(g @ v), rel=1e-7)
    for j in rng.choice(flat.size, size=6, replace=False):
        e = np.zeros_like(flat)
        e[j] = h
        fd = (_weighted_objective(cfg, flat + e, idx, tgt, tb, w)
              - _weighted_objective(cfg, flat - e, idx, tgt, tb, w)) / (2 * h)
        assert fd == pytest.approx(g[j], rel=1e-6, abs=1e-10)


def test_weighted_gradient_special_cases():
    """Unit weights give the unweighted gradient bit for bit; zero weight on
    a set of tokens equals ignoring those targets, rescaled by the changed
    count; the gradient is linear in the weights."""
    cfg = MICRO
    flat, p = _micro_params(seed=24)
    idx, tgt = synthdata.make_tokens(cfg)
    tb = synthdata.make_token_bytes(cfg)
    plain = np.concatenate(_flat(oracle.train_step(cfg, p, idx, tgt, tb)["grads"], cfg))
    ones = np.concatenate(_flat(oracle.train_step(cfg, p, idx, tgt, tb, token_weights=np.ones(tgt.shape))["grads"],
                                cfg))
    np.testing.assert_array_equal(plain, ones)
    keep = np.ones(tgt.shape)
    keep[1, :5] = 0.0
    keep[0, 7] = 0.0
    zeroed = np.concatenate(_flat(oracle.train_step(cfg, p, idx, tgt, tb, token_weights=keep)["grads"], cfg))
    masked_tgt = np.where(keep > 0, tgt, -1)
    masked = np.concatenate(_flat(oracle.train_step(cfg, p, idx, masked_tgt, tb)["grads"], cfg))
    n_all, n_kept = tgt.size, int(keep.sum())
    np.testing.assert_allclose(zeroed, masked * n_kept / n_all, rtol=1e-12, atol=1e-15)
    w1, w2 = _rng(25).standard_normal(tgt.shape), _rng(26).standard_normal(tgt.shape)
    g1, g2, g12 = (np.concatenate(_flat(oracle.train_step(cfg, p, idx, tgt, tb, token_weights=w)["grads"], cfg))
                   for w in (w1, w2, w1 + w2))
    np.testing.assert_allclose(g12, g1 + g2, rtol=1e-10, atol=1e-14)
    s, m = oracle.weighted_loss(np.ones(tgt.shape), tgt, w1)
    assert s == pytest.approx(w1.sum()) and m == pytest.approx(w1.sum() / tgt.size)


# --------------------------------------------------------------------------
# sampling the next token
# --------------------------------------------------------------------------
def test_sample_greedy_and_top1():
    z = _rng(31).standard_normal(500)
    z[123] = 9.0
    assert oracle.sample_next(z, 0.0, 0, 0.7) == 123
    for u in (0.0, 0.5, 0.999):
        assert oracle.sample_next(z, 1.3, 1, u) == 123


@pytest.mark.parametrize("temperature,top_k", [(1.0, 0), (0.7, 0), (1.5, 10)])
def test_sample_frequencies_on_a_uniform_grid(temperature, top_k):
    """Inverse CDF on the grid u_j = (j + 1/2) / N hits each token with
    frequency equal to its probability to within 1/N; the probabilities are
    scipy's softmax of z / temperature over the kept tokens."""
    from scipy.special import softmax
    z = _rng(32).standard_normal(40) * 2.0
    N = 20000
    counts = np.bincount([oracle.sample_next(z, temperature, top_k, (j + 0.5) / N) for j in range(N)],
                         minlength=z.size)
    keep = np.ones(z.size, dtype=bool) if top_k == 0 else z >= np.sort(z)[::-1][top_k - 1]
    p = np.zeros(z.size)
    p[keep] = softmax(z[keep] / temperature)
    assert np.abs(counts / N - p).max() <= 1.0 / N + 1e-12
    assert not np.any(counts[~keep])


def test_sample_top_k_keeps_ties():
    z = np.array([0.0, 3.0, 1.0, 3.0, 2.0, 2.0, -1.0])
    drawn = {oracle.sample_next(z, 1.0, 3, (j + 0.5) / 1000) for j in range(1000)}
    assert drawn == {1, 3, 4, 5}           # the two 2.0s tie for third place

