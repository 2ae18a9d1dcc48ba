"""Host-side checks of the C ABI that need no GPU: the library loads, every
function include/*.h declares is exported, the flat parameter layout agrees
with the seeded generators' layout, and invalid arguments are rejected before
any HIP call."""
import ctypes
import glob
import os
import re

import pytest

import synthdata
import decoder_only_transformer_d20_amd as nc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        txt = open(h).read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        names |= set(re.findall(r"\b(nc_[a-z0-9_]+)\s*\(", txt))
    return names


def test_library_exports_every_declared_function():
    L = ctypes.CDLL(nc.LIB_PATH)
    declared = _declared_functions()
    assert len(declared) >= 20
    missing = [n for n in sorted(declared) if not hasattr(L, n)]
    assert not missing, missing
    # and the binding wraps every one of them
    assert declared <= set(nc._SIGS), sorted(declared - set(nc._SIGS))


@pytest.mark.parametrize("name", list(synthdata.CONFIGS))
def test_param_layout_matches_generators(name):
    cfg = synthdata.get_config(name)
    assert nc.param_count(cfg) == synthdata.param_count(cfg)
    for tname, layer, r, c, off in synthdata.param_layout(cfg):
        assert nc.param_offset(cfg, tname, max(layer, 0)) == (off, r, c), (tname, layer)


def test_d20_param_count_exact():
    assert nc.param_count(synthdata.get_config("d20")) == 560_988_160


@pytest.mark.parametrize("name", list(synthdata.CONFIGS))
def test_workspace_is_positive_and_fits_hbm(name):
    cfg = synthdata.get_config(name)
    ws = nc.workspace_bytes(cfg)
    assert 0 < ws < 200 * 2 ** 30
    if name == "d20":
        # the saved activations dominate: ~1.7 GB per layer in bf16
        assert ws > 20 * 1.6e9


def _cfg(**kw):
    c = nc.make_config(synthdata.get_config("small"))
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,status", [
    ("d_model", 250, -2), ("head_dim", 100, -2), ("n_head", 3, -2), ("seq_len", 100, -2),
    ("n_layer", 0, -2), ("vocab", 0, -2), ("dtype", 7, -1), ("flags", 64, -1), ("rms_eps", -1.0, -1),
])
def test_invalid_configs_rejected(field, value, status):
    c = _cfg(**{field: value})
    assert nc.lib().nc_param_count(ctypes.byref(c)) == status
    assert nc.lib().nc_workspace_bytes(ctypes.byref(c)) == status


def test_block_only_rules():
    c = nc.make_config(synthdata.get_config("block"))
    assert c.flags & nc.FLAG_BLOCK_ONLY
    assert nc.param_count(c) == 12 * 1280 * 1280
    c.n_layer = 2
    assert nc.lib().nc_param_count(ctypes.byref(c)) == -2
    with pytest.raises(nc.NcError):
        nc.param_offset(synthdata.get_config("block"), "E")


def test_init_checks_before_any_hip_call():
    L = nc.lib()
    c = _cfg()
    h = ctypes.c_void_p()
    need = nc.workspace_bytes(c)
    assert L.nc_init(ctypes.byref(c), None, need, None, ctypes.byref(h)) == -1       # null workspace
    assert L.nc_init(ctypes.byref(c), 256, need - 1, None, ctypes.byref(h)) == -3    # too small
    assert L.nc_init(ctypes.byref(c), 256 + 8, need, None, ctypes.byref(h)) == -3    # misaligned
    assert L.nc_init(ctypes.byref(c), 256, need, None, None) == -1                   # no out pointer
    assert h.value is None


def test_calls_on_null_context_rejected():
    L = nc.lib()
    assert L.nc_forward(None, 1, 1, 1, None) == -1
    assert L.nc_forward_eval(None, 1, 1, 1, None) == -1
    assert L.nc_backward(None, 1, 1, 0) == -1
    assert L.nc_loss_bpb(None, 1, 1) == -1
    assert L.nc_block_forward(None, 1, 1, 2) == -1
    h = nc.NcOptimHparams()
    assert L.nc_optimizer_step(None, 16, 16, 16, 16, 256, ctypes.byref(h)) == -1
    assert L.nc_backward_weighted(None, 1, 1, 0, 1) == -1
    assert L.nc_loss_weighted(None, 1, 1) == -1
    assert L.nc_last_error(None) == b"null context"


def test_ops_reject_bad_shapes_before_launch():
    L = nc.lib()
    # M not a multiple of 64
    assert L.nc_op_matmul(1, 0, 0, 100, 64, 64, 1, 1, 1, 1, 1, None, 0, None) == -2
    # the matrix-core kernel's rounded output must be 16-byte aligned
    assert L.nc_op_matmul(1, 0, 0, 128, 128, 64, 256, 256, 258, 0, 1, None, 0, None) == -6
    # split-K without partial buffer / with a stored (non-fp32) output
    assert L.nc_op_matmul(1, 0, 0, 64, 64, 128, 1, 1, 1, 1, 2, None, 0, None) == -1
    assert L.nc_op_matmul(1, 0, 0, 64, 64, 128, 1, 1, 1, 0, 2, 1, 0, None) == -1
    assert L.nc_op_rmsnorm_fwd(1, 4, 100, 1e-6, 1, 1, 1, None) == -2
    assert L.nc_op_attention_fwd(1, 1, 100, 1, 128, 1, 1, 1, 0, None) == -2
    assert L.nc_op_attention_fwd(5, 1, 64, 1, 128, 1, 1, 1, 0, None) == -1
    assert L.nc_op_head_scratch_bytes(1, 128, 64, 100, 0) == -2
    # embedding gradient: sizes, then a missing scratch buffer
    assert L.nc_op_embed_bwd_scratch_bytes(0, 64) == -2
    assert L.nc_op_embed_bwd_scratch_bytes(10, 100) == -2
    assert L.nc_op_mfma_loop(0, 4, 1, None) == -2
    assert L.nc_op_mfma_loop(10, 0, 1, None) == -2
    assert L.nc_op_mfma_loop(10, 4, None, None) == -1
    assert L.nc_op_device_info(0, None, None, None, None) == -1
    assert L.nc_op_embed_bwd_scratch_bytes(10, 64) > 0
    assert L.nc_op_embed_bwd(1, 10, 100, 50, 1, 1, 1, 0, 1, None) == -2
    assert L.nc_op_embed_bwd(1, 10, 64, 50, 1, 1, 1, 0, None, None) == -1
    # stored-dS attention backward: scratch size (causal 64 x 128 tiles), then
    # a missing scratch buffer and a T that is not a multiple of 64
    assert L.nc_op_attention_ds_bytes(0, 128, 2) == -2
    assert L.nc_op_attention_ds_bytes(1, 100, 2) == -2
    assert L.nc_op_attention_ds_bytes(2, 2048, 10) == 2 * 10 * 16 * 17 * 64 * 128 * 2
    assert L.nc_op_attention_ds_bytes(1, 192, 1) == 2 * 3 * 64 * 128 * 2
    assert L.nc_op_attention_bwd_ds(1, 128, 1, 128, 1, 1, 1, 1, 1, 1, None, None, None) == -1
    assert L.nc_op_attention_bwd_ds(1, 100, 1, 128, 1, 1, 1, 1, 1, 1, None, 1, None) == -2
    # a batch row's qkv block of 2^31 bytes or more is beyond the matrix-core
    # kernels' 32-bit tile addressing: unsupported, reported before any launch
    assert L.nc_op_attention_fwd(1, 1, 1 << 19, 10, 128, 1, 1, 1, 0, None) == -6
    assert L.nc_op_attention_bwd_ds(1, 1 << 19, 10, 128, 1, 1, 1, 1, 1, 1, None, 1, None) == -6


def test_status_strings():
    assert nc.status_string(0) == "ok"
    assert "workspace" in nc.status_string(-3)
    assert nc.status_string(-99) == "unknown status"


def test_flop_formula_d20():
    from decoder_only_transformer_d20_amd.flops import flops_per_token, flops_per_step
    cfg = synthdata.get_config("d20")
    assert flops_per_token(cfg) == pytest.approx(3.492e9, rel=1e-3)
    assert flops_per_step(cfg) == pytest.approx(2.288e14, rel=1e-3)


# --------------------------------------------------------------------------
# optimiser step: host-only queries
# --------------------------------------------------------------------------
@pytest.mark.parametrize("it,num_iters,n_micro", [(0, 1000, 1), (150, 1000, 8), (850, 1000, 2), (999, 1000, 1),
                                                  (1000, 1000, 1), (7, 10, 4)])
def test_optim_default_matches_oracle_schedule(it, num_iters, n_micro):
    """nc_optim_default (host C) against the oracle's schedule and
    defaults, at d20 width."""
    from oracle import optim
    cfg = synthdata.get_config("d20")
    h = nc.optim_default(cfg, it, num_iters, n_micro)
    w = optim.default_hparams(cfg.d_model, it, num_iters, n_micro)
    for f in ("grad_scale", "lr_embed", "lr_unembed", "beta1", "beta2", "eps", "weight_decay", "lr_matrix",
              "momentum"):
        assert getattr(h, f) == pytest.approx(w[f], rel=1e-6, abs=1e-12), f
    assert h.adam_step == w["adam_step"] and h.nesterov == 1 and h.ns_steps == w["ns_steps"]
    assert (h.ns_a, h.ns_b, h.ns_c) == pytest.approx(w["ns_coeffs"], rel=1e-6)


def test_optim_sizes():
    cfg = synthdata.get_config("d20")
    P = synthdata.param_count(cfg)
    assert nc.optim_state_bytes(cfg) == 4 * (P + 2 * cfg.vocab * cfg.d_model)
    blk = synthdata.get_config("block")
    assert nc.optim_state_bytes(blk) == 4 * synthdata.param_count(blk)
    # Newton-Schulz operands batched per shape group: two ping-pong copies
    # of the 40 d x 4d matrices (W1 transposed, W2), two d x d products for
    # each of the 80 square ones, and 4 KB of partial sums per matrix
    es = 2
    assert nc.optim_scratch_bytes(cfg) == 80 * 4096 + 2 * 40 * 5120 * 1280 * es + 2 * 80 * 1280 * 1280 * es
    with pytest.raises(nc.NcError):
        nc.optim_default(cfg, 5, 4, 1)          # it past num_iters
    with pytest.raises(nc.NcError):
        nc.optim_default(cfg, 0, 10, 0)         # no micro-batch


def test_inference_sizes_and_null_context():
    cfg = synthdata.get_config("d20")
    # K and V per layer: [max_batch][max_len][d] bf16
    assert nc.kv_cache_bytes(cfg, 4, 2048) == 2 * 20 * 4 * 2048 * 1280 * 2
    assert nc.decode_scratch_bytes(cfg, 4, 2048) > 0
    with pytest.raises(nc.NcError):
        nc.kv_cache_bytes(cfg, 17, 2048)          # more sequences than one decode step takes
    with pytest.raises(nc.NcError):
        nc.kv_cache_bytes(synthdata.get_config("block"), 1, 64)
    L = nc.lib()
    assert L.nc_prefill(None, 1, 1, 1, 1, 1, 1, 64, 1) == -1
    assert L.nc_decode(None, 1, 1, 1, 0, 1, 1, 64, 256, 1) == -1
    # nc_sample checks its arguments before any launch
    assert L.nc_sample(None, 1, 8, 1.0, 0, 1, 1, None) == -1
    assert L.nc_sample(16, 1, 8, -1.0, 0, 16, 16, None) == -1
    assert L.nc_sample(16, 1, 8, 1.0, -2, 16, 16, None) == -1
    assert L.nc_sample(16, 0, 8, 1.0, 0, 16, 16, None) == -2
    assert L.nc_sample_parallel(None, 1, 8, 1.0, 0, 1, 1, 256, None) == -1
    assert L.nc_sample_parallel(16, 1, 8, 1.0, 0, 16, 16, None, None) == -1
    assert L.nc_sample_parallel(16, 1, 8, -1.0, 0, 16, 16, 256, None) == -1
    assert L.nc_sample_parallel(16, 1, 70000, 1.0, 0, 16, 16, 256, None) == -2
    assert L.nc_sample_parallel(16, 1, 8, 1.0, 0, 16, 16, 257, None) == -3
    assert L.nc_sample_scratch_bytes(0, 8) == -2 and L.nc_sample_scratch_bytes(1, 65537) == -2
    assert L.nc_sample_scratch_bytes(16, 65536) >= 16 * 64 * 256 * 4
