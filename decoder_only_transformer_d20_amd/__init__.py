"""MI355X (gfx950) forward/backward library for the nanochat d20 decoder-only
Transformer: Python binding of ``libnc.so`` (include/nc.h, include/nc_ops.h).

The binding only marshals arguments: every step of the training step runs in
the library's HIP kernels.  PyTorch, when used (``Session``), only provides
device memory and the current stream.  If the library has not been built,
loading fails with an error; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "lib", "NcConfig", "NcError", "Context", "Session", "make_config", "param_count",
    "param_offset", "workspace_bytes", "status_string", "ops", "LIB_PATH",
    "DTYPE_F32", "DTYPE_BF16", "FLAG_BLOCK_ONLY", "FLAG_PORTABLE_KERNELS",
    "NcOptimHparams", "optim_default", "optim_state_bytes", "optim_scratch_bytes",
    "kv_cache_bytes", "decode_scratch_bytes", "decode_static_max_bytes", "sample",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnc.so")

DTYPE_F32, DTYPE_BF16 = 0, 1
FLAG_BLOCK_ONLY, FLAG_PORTABLE_KERNELS = 1, 2
TENSOR_IDS = {"E": 0, "Wq": 1, "Wk": 2, "Wv": 3, "Wo": 4, "W1": 5, "W2": 6, "U": 7}
# nc.h NC_TRACE_* in order; every family but attn_bwd is a single kernel
TRACE_FAMILIES = ["gemm_qkv_rope", "gemm_residual", "gemm_relu2", "gemm_head_lse", "gemm_head_dz", "gemm_dgrad",
                  "gemm_dgrad_relu2", "gemm_wgrad", "attn_fwd", "attn_bwd"]
SINGLE_KERNEL_FAMILIES = TRACE_FAMILIES[:-1]
# NC_TRACE_OPTIM_*: launches inside nc_optimizer_step
OPTIM_TRACE_FAMILIES = ["optim_ns", "optim_adamw"]


class NcConfig(ctypes.Structure):
    _fields_ = [
        ("n_layer", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_head", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("vocab", ctypes.c_int32),
        ("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("rope_base", ctypes.c_float),
        ("rms_eps", ctypes.c_float), ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
    ]


class NcOptimHparams(ctypes.Structure):
    """nc_optim_hparams (include/nc.h)."""
    _fields_ = [
        ("grad_scale", ctypes.c_float), ("lr_embed", ctypes.c_float), ("lr_unembed", ctypes.c_float),
        ("beta1", ctypes.c_float), ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
        ("weight_decay", ctypes.c_float), ("adam_step", ctypes.c_int32), ("lr_matrix", ctypes.c_float),
        ("momentum", ctypes.c_float), ("nesterov", ctypes.c_int32), ("ns_steps", ctypes.c_int32),
        ("ns_a", ctypes.c_float), ("ns_b", ctypes.c_float), ("ns_c", ctypes.c_float),
    ]


class NcError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str = ""):
        self.status = status
        msg = f"{what}: {status_string(status)} ({status})"
        if detail:
            msg += f": {detail}"
        super().__init__(msg)


_lib = None
_P = ctypes.c_void_p
_I32, _I64, _F32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_SIGS = {
    "nc_param_count": (_I64, [ctypes.POINTER(NcConfig)]),
    "nc_param_offset": (ctypes.c_int, [ctypes.POINTER(NcConfig), _I32, _I32, ctypes.POINTER(_I64),
                                       ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "nc_workspace_bytes": (_I64, [ctypes.POINTER(NcConfig)]),
    "nc_optim_default": (ctypes.c_int, [ctypes.POINTER(NcConfig), _I64, _I64, _I32, ctypes.POINTER(NcOptimHparams)]),
    "nc_optim_state_bytes": (_I64, [ctypes.POINTER(NcConfig)]),
    "nc_optim_scratch_bytes": (_I64, [ctypes.POINTER(NcConfig)]),
    "nc_optimizer_step": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.POINTER(NcOptimHparams)]),
    "nc_backward_weighted": (ctypes.c_int, [_P, _P, _P, _I32, _P]),
    "nc_kv_cache_bytes": (_I64, [ctypes.POINTER(NcConfig), _I32, _I32]),
    "nc_sample": (ctypes.c_int, [_P, _I32, _I32, _F32, _I32, _P, _P, _P]),
    "nc_sample_scratch_bytes": (_I64, [_I32, _I32]),
    "nc_sample_parallel": (ctypes.c_int, [_P, _I32, _I32, _F32, _I32, _P, _P, _P, _P]),
    "nc_decode_scratch_bytes": (_I64, [ctypes.POINTER(NcConfig), _I32, _I32]),
    "nc_prefill": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _P, _I32, _I32, _P]),
    "nc_decode": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _P, _I32, _I32, _P, _P]),
    "nc_decode_static_max_bytes": (_I64, []),
    "nc_decode_static": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _P, _I32, _I32, _P]),
    "nc_loss_weighted": (ctypes.c_int, [_P, _P, _P]),
    "nc_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "nc_init": (ctypes.c_int, [ctypes.POINTER(NcConfig), _P, ctypes.c_size_t, _P, ctypes.POINTER(_P)]),
    "nc_set_stream": (ctypes.c_int, [_P, _P]),
    "nc_destroy": (None, [_P]),
    "nc_last_error": (ctypes.c_char_p, [_P]),
    "nc_fallback_count": (ctypes.c_int, [_P, ctypes.POINTER(_I64), _I32]),
    "nc_forward": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "nc_forward_eval": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "nc_loss_bpb": (ctypes.c_int, [_P, _P, _P]),
    "nc_backward": (ctypes.c_int, [_P, _P, _P, _I32]),
    "nc_block_forward": (ctypes.c_int, [_P, _P, _P, _P]),
    "nc_block_backward": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32]),
    "nc_trace_enable": (ctypes.c_int, [_P, _I32]),
    "nc_trace_read": (ctypes.c_int, [_P, ctypes.POINTER(_I64), ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]),
    "nc_op_matmul": (ctypes.c_int, [_I32, _I32, _I32, _I64, _I64, _I64, _P, _P, _P, _I32, _I32, _P, _I32, _P]),
    "nc_op_matmul_batched": (ctypes.c_int, [_I32, _I32, _I32, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _P,
                                            _I64, _F32, _F32, _I32, _I32, _P]),
    "nc_op_rmsnorm_fwd": (ctypes.c_int, [_I32, _I64, _I32, _F32, _P, _P, _P, _P]),
    "nc_op_rmsnorm_bwd": (ctypes.c_int, [_I32, _I64, _I32, _P, _P, _P, _P, _I32, _P]),
    "nc_op_rope_table": (ctypes.c_int, [_I32, _I32, _F32, _P, _P]),
    "nc_op_mfma_loop": (ctypes.c_int, [_I64, _I32, _P, _P]),
    "nc_op_device_info": (ctypes.c_int, [_I32] + [ctypes.POINTER(_I32)] * 4),
    "nc_op_attention_fwd": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, _P, _P, _P, _I32, _P]),
    "nc_op_attention_bwd": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _I32, _P]),
    "nc_op_attention_bwd_ds": (ctypes.c_int, [_I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "nc_op_attention_ds_bytes": (_I64, [_I32, _I32, _I32]),
    "nc_op_embed_fwd": (ctypes.c_int, [_I32, _I64, _I32, _I32, _P, _P, _P, _P]),
    "nc_op_embed_bwd_scratch_bytes": (_I64, [_I64, _I32]),
    "nc_op_embed_bwd": (ctypes.c_int, [_I32, _I64, _I32, _I32, _P, _P, _P, _I32, _P, _P]),
    "nc_op_head_scratch_bytes": (_I64, [_I32, _I64, _I32, _I32, _I32]),
    "nc_op_head_ce_fwd": (ctypes.c_int, [_I32, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _I32, _P]),
    "nc_op_head_gemm_lse": (ctypes.c_int, [_I32, _I64, _I32, _I32, _P, _P, _P, _P, _P]),
}


def lib():
    """Load libnc.so (built in-tree by ``_build.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run decoder_only_transformer_d20_amd._build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().nc_status_string(int(status)).decode()


def _check(status: int, what: str, ctx=None):
    if status != 0:
        detail = lib().nc_last_error(ctx).decode() if ctx else ""
        raise NcError(status, what, detail)


def make_config(cfg, portable: bool = False) -> NcConfig:
    """NcConfig from any object with the model's attribute names
    (n_layer, d_model, n_head, head_dim, d_ff, vocab, batch, seq_len, dtype
    "f32"/"bf16", block_only, rope_base, rms_eps)."""
    flags = (FLAG_BLOCK_ONLY if getattr(cfg, "block_only", False) else 0)
    flags |= FLAG_PORTABLE_KERNELS if portable else 0
    dt = cfg.dtype
    dt = {"f32": DTYPE_F32, "bf16": DTYPE_BF16}.get(dt, dt)
    return NcConfig(cfg.n_layer, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.d_ff, cfg.vocab, cfg.batch,
                    cfg.seq_len, float(getattr(cfg, "rope_base", 10000.0)), float(getattr(cfg, "rms_eps", 1e-6)),
                    int(dt), flags)


def _c(cfg):
    return cfg if isinstance(cfg, NcConfig) else make_config(cfg)


def param_count(cfg) -> int:
    n = lib().nc_param_count(ctypes.byref(_c(cfg)))
    _check(0 if n >= 0 else n, "nc_param_count")
    return n


def param_offset(cfg, tensor, layer: int = 0):
    t = TENSOR_IDS[tensor] if isinstance(tensor, str) else int(tensor)
    off, r, c = _I64(), _I64(), _I64()
    _check(lib().nc_param_offset(ctypes.byref(_c(cfg)), t, layer, ctypes.byref(off), ctypes.byref(r),
                                 ctypes.byref(c)), "nc_param_offset")
    return off.value, r.value, c.value


def workspace_bytes(cfg) -> int:
    n = lib().nc_workspace_bytes(ctypes.byref(_c(cfg)))
    _check(0 if n >= 0 else n, "nc_workspace_bytes")
    return n


def optim_default(cfg, it: int, num_iters: int, n_micro: int = 1) -> NcOptimHparams:
    """nc_optim_default: the step's default hyperparameters (host-only)."""
    h = NcOptimHparams()
    _check(lib().nc_optim_default(ctypes.byref(_c(cfg)), int(it), int(num_iters), int(n_micro), ctypes.byref(h)),
           "nc_optim_default")
    return h


def optim_state_bytes(cfg) -> int:
    n = lib().nc_optim_state_bytes(ctypes.byref(_c(cfg)))
    _check(0 if n >= 0 else n, "nc_optim_state_bytes")
    return n


def optim_scratch_bytes(cfg) -> int:
    n = lib().nc_optim_scratch_bytes(ctypes.byref(_c(cfg)))
    _check(0 if n >= 0 else n, "nc_optim_scratch_bytes")
    return n


def sample(logits, n: int, V: int, temperature: float, top_k: int, u, out, stream=None):
    """nc_sample: next token per row of fp32 logits [n][V] from uniforms u [n]."""
    _check(lib().nc_sample(_ptr(logits), int(n), int(V), float(temperature), int(top_k), _ptr(u), _ptr(out),
                           _ptr(stream)), "nc_sample")


def sample_scratch_bytes(n: int, V: int) -> int:
    r = lib().nc_sample_scratch_bytes(int(n), int(V))
    _check(0 if r >= 0 else r, "nc_sample_scratch_bytes")
    return r


def sample_parallel(logits, n: int, V: int, temperature: float, top_k: int, u, out, scratch, stream=None):
    """nc_sample_parallel: nc_sample over ceil(V/1024) workgroups per row;
    scratch: device buffer of sample_scratch_bytes(n, V) bytes, 256-aligned."""
    _check(lib().nc_sample_parallel(_ptr(logits), int(n), int(V), float(temperature), int(top_k), _ptr(u), _ptr(out),
                                    _ptr(scratch), _ptr(stream)), "nc_sample_parallel")


def kv_cache_bytes(cfg, max_batch: int, max_len: int) -> int:
    n = lib().nc_kv_cache_bytes(ctypes.byref(_c(cfg)), int(max_batch), int(max_len))
    _check(0 if n >= 0 else n, "nc_kv_cache_bytes")
    return n


def decode_scratch_bytes(cfg, max_batch: int, max_len: int) -> int:
    n = lib().nc_decode_scratch_bytes(ctypes.byref(_c(cfg)), int(max_batch), int(max_len))
    _check(0 if n >= 0 else n, "nc_decode_scratch_bytes")
    return n


def decode_static_max_bytes() -> int:
    """Size of the static scratch nc_decode_static uses (host-only query)."""
    return lib().nc_decode_static_max_bytes()


def _ptr(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


class Context:
    """An nc_ctx over caller-provided device pointers (ints or tensors)."""

    def __init__(self, cfg, workspace, ws_bytes: int, stream=None):
        self.cfg = _c(cfg)
        self._ws = workspace          # keep the owner alive
        h = _P()
        _check(lib().nc_init(ctypes.byref(self.cfg), _ptr(workspace), int(ws_bytes), _ptr(stream), ctypes.byref(h)),
               "nc_init")
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            lib().nc_destroy(self.h)
            self.h = None

    def __del__(self):
        self.close()

    def set_stream(self, stream):
        _check(lib().nc_set_stream(self.h, _ptr(stream)), "nc_set_stream", self.h)

    def forward(self, params, idx, targets, ce_out=None):
        _check(lib().nc_forward(self.h, _ptr(params), _ptr(idx), _ptr(targets), _ptr(ce_out)), "nc_forward", self.h)

    def forward_eval(self, params, idx, targets, ce_out=None):
        """nc_forward_eval: the forward for evaluation (no logits kept)."""
        _check(lib().nc_forward_eval(self.h, _ptr(params), _ptr(idx), _ptr(targets), _ptr(ce_out)),
               "nc_forward_eval", self.h)

    def loss_bpb(self, token_bytes, out):
        _check(lib().nc_loss_bpb(self.h, _ptr(token_bytes), _ptr(out)), "nc_loss_bpb", self.h)

    def backward(self, params, grads, accumulate: bool = False):
        _check(lib().nc_backward(self.h, _ptr(params), _ptr(grads), int(bool(accumulate))), "nc_backward", self.h)

    def backward_weighted(self, params, grads, token_weights, accumulate: bool = False):
        """nc_backward_weighted: gradient of sum_t w_t ce[t] / n_valid."""
        _check(lib().nc_backward_weighted(self.h, _ptr(params), _ptr(grads), int(bool(accumulate)),
                                          _ptr(token_weights)), "nc_backward_weighted", self.h)

    def loss_weighted(self, token_weights, out):
        """nc_loss_weighted: out[0] = sum_t w_t ce[t], out[1] = that / n_valid."""
        _check(lib().nc_loss_weighted(self.h, _ptr(token_weights), _ptr(out)), "nc_loss_weighted", self.h)

    def prefill(self, params, idx, prompt_len: int, nseq: int, kv_cache, max_batch: int, max_len: int, logits):
        """nc_prefill: the prompt's K, V into the cache, last-position logits."""
        _check(lib().nc_prefill(self.h, _ptr(params), _ptr(idx), int(prompt_len), int(nseq), _ptr(kv_cache),
                                int(max_batch), int(max_len), _ptr(logits)), "nc_prefill", self.h)

    def decode(self, params, tokens, nseq: int, pos: int, kv_cache, max_batch: int, max_len: int, scratch, logits):
        """nc_decode: one token per sequence at position pos, next-token logits."""
        _check(lib().nc_decode(self.h, _ptr(params), _ptr(tokens), int(nseq), int(pos), _ptr(kv_cache),
                               int(max_batch), int(max_len), _ptr(scratch), _ptr(logits)), "nc_decode", self.h)

    def decode_static(self, params, tokens, nseq: int, pos: int, kv_cache, max_batch: int, max_len: int, logits):
        """nc_decode_static: nc_decode with the library's static device
        scratch (no scratch argument, nothing allocated)."""
        _check(lib().nc_decode_static(self.h, _ptr(params), _ptr(tokens), int(nseq), int(pos), _ptr(kv_cache),
                                      int(max_batch), int(max_len), _ptr(logits)), "nc_decode_static", self.h)

    def fallback_count(self, reset: bool = False) -> int:
        """nc_fallback_count: bf16 launches that took a portable kernel."""
        n = _I64()
        _check(lib().nc_fallback_count(self.h, ctypes.byref(n), int(bool(reset))), "nc_fallback_count", self.h)
        return n.value

    def trace_enable(self, family):
        """Time launches of one kernel family (a name from TRACE_FAMILIES or
        its index; None disables)."""
        names = TRACE_FAMILIES + OPTIM_TRACE_FAMILIES
        f = -1 if family is None else (names.index(family) if isinstance(family, str) else int(family))
        _check(lib().nc_trace_enable(self.h, f), "nc_trace_enable", self.h)

    def trace_read(self):
        """(launches, total ms, total algorithmic FLOPs, total algorithmic bytes)."""
        n, ms, fl, by = _I64(), ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        _check(lib().nc_trace_read(self.h, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(fl), ctypes.byref(by)),
               "nc_trace_read", self.h)
        return n.value, ms.value, fl.value, by.value

    def optimizer_step(self, master, params, grads, state, scratch, hparams: NcOptimHparams):
        """nc_optimizer_step: AdamW on E and U, Muon on every block matrix."""
        _check(lib().nc_optimizer_step(self.h, _ptr(master), _ptr(params), _ptr(grads), _ptr(state), _ptr(scratch),
                                       ctypes.byref(hparams)), "nc_optimizer_step", self.h)

    def block_forward(self, params, x, y):
        _check(lib().nc_block_forward(self.h, _ptr(params), _ptr(x), _ptr(y)), "nc_block_forward", self.h)

    def block_backward(self, params, dy, dx, dparams, accumulate: bool = False):
        _check(lib().nc_block_backward(self.h, _ptr(params), _ptr(dy), _ptr(dx), _ptr(dparams),
                                       int(bool(accumulate))), "nc_block_backward", self.h)


class Session(Context):
    """Context whose workspace is a torch CUDA byte tensor and whose stream is
    torch's current stream at construction (torch provides memory and the
    stream only)."""

    def __init__(self, cfg, portable: bool = False, device="cuda"):
        import torch
        c = make_config(cfg, portable=portable) if not isinstance(cfg, NcConfig) else cfg
        nbytes = workspace_bytes(c)
        ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        base = ws.data_ptr()
        aligned = (base + 255) // 256 * 256
        self.stream = torch.cuda.current_stream(device)
        super().__init__(c, aligned, nbytes, self.stream.cuda_stream)
        self._ws = ws


class _Ops:
    """Component entry points (include/nc_ops.h); pointer args are tensors or ints."""

    def __getattr__(self, name):
        f = getattr(lib(), "nc_op_" + name)

        def call(*args):
            conv = [(_ptr(a) if (a is None or hasattr(a, "data_ptr")) else a) for a in args]
            st = f(*conv)
            if name.endswith("_bytes"):
                _check(0 if st >= 0 else st, "nc_op_" + name)
                return st
            _check(st, "nc_op_" + name)
            return st

        return call


ops = _Ops()
