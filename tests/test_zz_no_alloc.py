"""nc_decode_static, the decode step that allocates nothing (its scratch is
a static device array of the library), against nc_decode with a caller
scratch: the same kernels, so logits and the appended cache entries must
agree bit for bit.  Two calls in a row, the second smaller (fewer
sequences, one more cached position), so the second runs over what the
first left in the shared array."""
import numpy as np
import pytest

import synthdata
from _util import dev, empty, host, zeros

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import decoder_only_transformer_d20_amd as nc  # noqa: E402


def test_decode_static_matches_decode_on_two_calls():
    cfg = synthdata.get_config("small")
    params = synthdata.make_params(cfg)
    T0, mb, pad = 100, 4, 128
    pcfg = cfg.with_(batch=1, seq_len=pad)
    ml = T0 + 8
    sess = nc.Session(pcfg)
    P = dev(params, cfg.dtype)
    rng = np.random.default_rng(77)
    idx = np.concatenate([rng.integers(0, cfg.vocab, T0), np.zeros(pad - T0, np.int64)]).astype(np.int32)
    kv_a = zeros((nc.kv_cache_bytes(pcfg, mb, ml) // 4,))
    l0 = empty((cfg.vocab,))
    sess.prefill(P, dev(idx), T0, mb, kv_a, mb, ml, l0)
    kv_b = kv_a.clone()
    scr = empty((nc.decode_scratch_bytes(pcfg, mb, ml) // 4 + 64,))
    sp = (scr.data_ptr() + 255) // 256 * 256
    for step, nseq in enumerate((4, 2)):
        tok = dev(rng.integers(0, cfg.vocab, nseq).astype(np.int32))
        la, lb = empty((nseq, cfg.vocab)), empty((nseq, cfg.vocab))
        sess.decode(P, tok, nseq, T0 + step, kv_a, mb, ml, sp, la)
        sess.decode_static(P, tok, nseq, T0 + step, kv_b, mb, ml, lb)
        torch.cuda.synchronize()
        a, b = host(la), host(lb)
        assert np.all(np.isfinite(a)), step
        np.testing.assert_array_equal(a, b, err_msg=f"call {step}")
        np.testing.assert_array_equal(host(kv_a), host(kv_b), err_msg=f"cache after call {step}")


def test_decode_static_rejects_a_call_beyond_its_maximum():
    """A call whose scratch would exceed the static array returns
    NC_ERR_WORKSPACE before any launch (the buffers are real and of the
    stated sizes all the same)."""
    cfg = synthdata.get_config("small").with_(batch=1, seq_len=64)
    sess = nc.Session(cfg)
    P = dev(synthdata.make_params(cfg), "bf16")
    nseq, pos = 16, 64600                  # attention partials alone: 16 x 2 x 1010 x 130 x 4 B > 16 MiB
    assert nc.decode_static_max_bytes() == 16 << 20
    assert nc.decode_scratch_bytes(cfg, nseq, pos + 1) > nc.decode_static_max_bytes()
    kv = empty((nc.kv_cache_bytes(cfg, nseq, pos + 1) // 4,))
    lg = empty((nseq, cfg.vocab))
    tok = dev(np.zeros(nseq, dtype=np.int32))
    with pytest.raises(nc.NcError) as e:
        sess.decode_static(P, tok, nseq, pos, kv, nseq, pos + 1, lg)
    assert e.value.status == -3
    assert "static maximum" in str(e.value)
