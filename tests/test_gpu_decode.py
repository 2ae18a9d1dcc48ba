"""KV-cache inference (nc_prefill, nc_decode) against the fp64 oracle.

Decoding is exact in the method: the logits decode produces at position t
are the logits the forward over the whole sequence gives at t (causal
attention), so the oracle is the pinned forward (oracle.model_forward_row)
run on each sequence's prompt + generated tokens.  The generated tokens are
fixed (teacher-forced), so every step is compared.

Bars: fp32 (tiny) max |dz| / max |z| <= 1e-4 per row.  bf16 (small, d20):
from an error model, not from the GPU's own numbers.  The library stores
every activation in bf16 (residual stream, norm outputs, q/k/v, attention
output, relu^2), so its logits differ from fp64 by the propagated storage
rounding.  tests/_util.logits_bf16_storage recomputes the logits on the CPU
with exactly that rounding (products exact) for the same sequence; per
position, the GPU's max |dz| must lie within 2x the model's max |dz| (plus
1e-3 of the row's largest logit), and its cosine distance 1 - cos within
2x the model's (plus 1e-5).  The factor 2 covers what the model leaves
out: fp32 accumulation order and rounding in the kernels' intermediates,
which differ from the model's exact products by far less than the storage
rounding itself."""
import numpy as np
import pytest

import oracle
import synthdata
from _util import cosine, dev, empty, host, zeros, logits_bf16_storage

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import decoder_only_transformer_d20_amd as nc  # noqa: E402


def _oracle_logits(cfg, params64, tokens):
    _, cache = oracle.model_forward_row(params64, np.asarray(tokens), np.zeros(len(tokens), dtype=np.int64), cfg)
    return cache["z"]


def _run(cfg, params, prompt, gen, nseq):
    """Prefill the prompt for nseq sequences, then decode gen[s][i] at
    position len(prompt) + i.  Returns (prefill logits [V], decode logits
    [steps][nseq][V])."""
    T0 = len(prompt)
    pad = (T0 + 63) // 64 * 64
    pcfg = cfg.with_(batch=1, seq_len=pad)
    steps = gen.shape[1]
    ml = T0 + steps
    sess = nc.Session(pcfg)
    P = dev(params, cfg.dtype)
    idx = np.concatenate([prompt, np.arange(pad - T0) % cfg.vocab]).astype(np.int32)
    kv = zeros((nc.kv_cache_bytes(pcfg, nseq, ml) // 4,))
    scr = empty((nc.decode_scratch_bytes(pcfg, nseq, ml) // 4 + 64,))
    sp = (scr.data_ptr() + 255) // 256 * 256
    l0 = empty((cfg.vocab,))
    sess.prefill(P, dev(idx), T0, nseq, kv, nseq, ml, l0)
    out = []
    for i in range(steps):
        li = empty((nseq, cfg.vocab))
        sess.decode(P, dev(gen[:, i].astype(np.int32)), nseq, T0 + i, kv, nseq, ml, sp, li)
        torch.cuda.synchronize()
        out.append(host(li))
    torch.cuda.synchronize()
    return host(l0), out


def _check(cfg, params, prompt, gen, nseq, bf16):
    l0, steps = _run(cfg, params, prompt, gen, nseq)
    p64 = synthdata.split_params(cfg, params.astype(np.float64))
    T0 = len(prompt)

    def ok(got, want, model, what):
        err = np.abs(got - want).max()
        if bf16:
            # bars from the bf16 storage error model of the same position
            m_err = np.abs(model - want).max()
            m_dist = 1.0 - cosine(model, want)
            bar = 2.0 * m_err + 1e-3 * np.abs(want).max()
            assert err <= bar, (what, err, m_err)
            assert 1.0 - cosine(got, want) <= 2.0 * m_dist + 1e-5, (what, cosine(got, want), 1.0 - m_dist)
        else:
            assert err <= 1e-4 * np.abs(want).max(), (what, err)

    for s in range(nseq):
        seq = np.concatenate([prompt, gen[s]])
        z = _oracle_logits(cfg, p64, seq)
        zm = logits_bf16_storage(cfg, p64, seq) if bf16 else z
        if s == 0:
            ok(l0, z[T0 - 1], zm[T0 - 1], "prefill")
        for i, li in enumerate(steps):
            ok(li[s], z[T0 + i], zm[T0 + i], ("decode", s, i))


def _tokens(cfg, T0, nseq, steps, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, cfg.vocab, T0), rng.integers(0, cfg.vocab, (nseq, steps))


def test_tiny_fp32_decode_matches_forward():
    """A 40-token prompt (padded to 64 for the prefill), three sequences,
    six steps."""
    cfg = synthdata.get_config("tiny")
    params = synthdata.make_params(cfg)
    prompt, gen = _tokens(cfg, 40, 3, 6, 51)
    _check(cfg, params, prompt, gen, 3, bf16=False)


@pytest.mark.parametrize("T0,nseq,steps", [(100, 4, 5), (255, 2, 3), (1, 1, 4), (1022, 2, 4)])
def test_small_bf16_decode_matches_forward(T0, nseq, steps):
    """bf16, including a one-token prompt, caches that cross 64-key chunk
    boundaries of the decode attention, and one of 1023 to 1026 keys (17
    chunks)."""
    cfg = synthdata.get_config("small")
    params = synthdata.make_params(cfg)
    prompt, gen = _tokens(cfg, T0, nseq, steps, 52 + T0)
    _check(cfg, params, prompt, gen, nseq, bf16=True)


@pytest.mark.parametrize("T0", [1, 100, 255, 300])
def test_prefill_runs_on_matrix_cores(T0):
    """A prompt padded to a multiple of 128 (the matrix-core products take
    128-row tiles) runs every product and attention call of the prefill on
    the matrix-core kernels: no launch falls back to the portable ones.
    (Attention alone takes any multiple of 64; see the attention op tests
    at T = 192 and 320.)"""
    cfg = synthdata.get_config("small")
    pad = (T0 + 127) // 128 * 128
    pcfg = cfg.with_(batch=1, seq_len=pad)
    sess = nc.Session(pcfg)
    P = dev(synthdata.make_params(cfg), "bf16")
    kv = zeros((nc.kv_cache_bytes(pcfg, 1, pad) // 4,))
    lg = empty((cfg.vocab,))
    sess.prefill(P, dev(np.zeros(pad, dtype=np.int32)), T0, 1, kv, 1, pad, lg)
    torch.cuda.synchronize()
    assert sess.fallback_count() == 0


def test_decode_rejects_bad_shapes():
    cfg = synthdata.get_config("small").with_(batch=1, seq_len=64)
    sess = nc.Session(cfg)
    params = synthdata.make_params(cfg)
    P = dev(params, "bf16")
    kv = zeros((nc.kv_cache_bytes(cfg, 2, 64) // 4,))
    scr = empty((nc.decode_scratch_bytes(cfg, 2, 64) // 4 + 64,))
    sp = (scr.data_ptr() + 255) // 256 * 256
    lg = empty((2, cfg.vocab))
    tok = dev(np.zeros(2, dtype=np.int32))
    for nseq, pos, mb, ml in ((3, 0, 2, 64), (1, 64, 2, 64), (0, 0, 2, 64), (1, 0, 17, 64)):
        with pytest.raises(nc.NcError) as e:
            sess.decode(P, tok, nseq, pos, kv, mb, ml, sp, lg)
        assert e.value.status == -2
    with pytest.raises(nc.NcError) as e:
        sess.prefill(P, dev(np.zeros(64, dtype=np.int32)), 65, 1, kv, 2, 64, lg)
    assert e.value.status == -2


def test_decode_bad_token_gives_nan_logits_for_its_sequence():
    """A token outside [0, V) is read nowhere: its sequence's logits are
    NaN, the other sequences' logits equal a run without it, bit for bit."""
    cfg = synthdata.get_config("small")
    params = synthdata.make_params(cfg)
    prompt, gen = _tokens(cfg, 60, 3, 1, 54)
    l0, good = _run(cfg, params, prompt, gen, 3)
    bad = gen.copy()
    bad[1, 0] = cfg.vocab + 11
    _, got = _run(cfg, params, prompt, bad, 3)
    assert np.all(np.isnan(got[0][1]))
    np.testing.assert_array_equal(got[0][[0, 2]], good[0][[0, 2]])


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_d20_decode_matches_forward():
    """The full d20 model: a 200-token prompt, two sequences, three steps."""
    cfg = synthdata.get_config("d20")
    params = synthdata.make_params(cfg)
    prompt, gen = _tokens(cfg, 200, 2, 3, 53)
    _check(cfg, params, prompt, gen, 2, bf16=True)


@pytest.mark.parametrize("parallel", [False, True])
@pytest.mark.parametrize("V,temperature,top_k", [(4096, 0.0, 0), (4096, 1.0, 0), (65536, 0.8, 50),
                                                 (65536, 1.0, 1), (1000, 1.3, 7), (65536, 1.0, 0),
                                                 (5000, 1.0, 256), (65536, 0.7, 300), (3000, 0.0, 5),
                                                 (2049, 1.0, 2049)])
def test_sample_matches_oracle(V, temperature, top_k, parallel):
    """nc_sample and nc_sample_parallel against oracle.sample_next on 64
    rows with the same uniforms, including a row of all-equal logits (top-k
    keeps every tie), a row with one dominant logit and a row whose largest
    logit repeats in several 1024-id blocks (the first id wins at
    temperature 0).  The GPU's weights are fp32 exponentials (relative error
    ~1e-7) summed in fp64, the oracle's fp64 throughout, so a draw may
    differ only where u * sum lies within 1e-6 of the total from a boundary
    of the inverse CDF; such a draw must still be a kept id next to the
    boundary."""
    rng = np.random.default_rng(60 + V + top_k)
    n = 64
    z = (rng.standard_normal((n, V)) * 3).astype(np.float32)
    z[5, :] = 0.25
    z[6, 17] = 40.0
    z[7, V - 1] = z[7, V // 2] = z[7, 3] = 30.0
    u = rng.random(n).astype(np.float32)
    out = empty((n,), "i32")
    if parallel:
        scr = empty((nc.sample_scratch_bytes(n, V) // 4 + 64,))
        sp = (scr.data_ptr() + 255) // 256 * 256
        nc.sample_parallel(dev(z), n, V, temperature, top_k, dev(u), out, sp)
    else:
        nc.sample(dev(z), n, V, temperature, top_k, dev(u), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    t32 = float(np.float32(temperature))
    for r in range(n):
        want = oracle.sample_next(z[r].astype(np.float64), t32, top_k, float(u[r]))
        if got[r] == want:
            continue
        zz = z[r].astype(np.float64)
        keep = np.ones(V, bool) if top_k in (0,) or top_k >= V else zz >= np.sort(zz)[::-1][top_k - 1]
        c = np.cumsum(np.where(keep, np.exp((zz - zz.max()) / t32), 0.0))
        assert keep[got[r]] and abs(c[min(got[r], want)] - float(u[r]) * c[-1]) <= 1e-6 * c[-1], (r, got[r], want)
    if temperature == 0.0:
        np.testing.assert_array_equal(got, np.argmax(z, axis=1))
    if top_k == 1:
        # one largest logit: top-1 is greedy; the all-equal row keeps every tie
        unique = (z == z.max(axis=1, keepdims=True)).sum(axis=1) == 1
        np.testing.assert_array_equal(got[unique], np.argmax(z, axis=1)[unique])
