"""Benchmark: one d20 training step (forward + loss/bpb + backward) per step on
one MI355X, through the C ABI (include/nc.h).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config d20|d30|block]
                    [--no-cpu-baseline] [--no-roofline] [--copy-calibration]
                    [--mfma-calibration] [--optimizer] [--decode [--decode-nseq 1,8,16]]
                    [--library-gemm]

Prints one JSON line.  `value` is training tokens/s of the whole job with
inputs already resident in HBM (host-to-device copies happen before timing);
MFU uses the FLOP convention of decoder_only_transformer_d20_amd.flops
against the bf16 dense MFMA peak of 2.5 PFLOP/s.

`roofline`: one untimed traced step per kernel family ranks the families by
time; during the timed steps the largest family's launches are bracketed by
HIP events on the library's stream (nc_trace_*), and `achieved` is its
algorithmic FLOPs per launch divided by its average launch time.
`traffic` is the HBM traffic per launch measured with rocprofv3 FETCH_SIZE /
WRITE_SIZE counters (calibrated against a plain device copy), reported only
while the measured kernel's source is unchanged.

`cpu_baseline`: the fp64 oracle (untuned) on the first --cpu-sample-tokens
(2048) tokens of row 0 -- forward, loss and backward -- on this host's cores.
`optimizer_step`: one Muon + AdamW step over every parameter, timed
separately (not part of `value`).

Other modes print their own JSON line and exit:
  --copy-calibration  a 1 GiB device-to-device copy (the reference kernel for
                      scaling the FETCH_SIZE / WRITE_SIZE counters)
  --mfma-calibration  the register-only MFMA loop's TFLOP/s
  --optimizer         the optimiser step alone, with its two kernel families
  --decode            KV-cache prefill + sampled decode, per batch size
  --library-gemm      nc_op_matmul next to torch.matmul (the vendor BLAS) on
                      the d20 product shapes
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "train tokens/s + MFU (fwd+bwd) on 1 MI355X, d20 at 32x2048 tok/step"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, TFLOP/s

# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
# on `python bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-roofline`,
# scaled by the counters' reading for --copy-calibration (see profiles/).
# Keyed by family; valid only for the recorded hash of the kernel source.
TRAFFIC = {
    # profiles/d20_step_hbm_traffic.md: 1.592 GB fetched + 0.134 GB written per dispatch
    "gemm_wgrad": {"bytes_per_launch": 1725486373, "source_hash": "ae9d0f9c7516286c"},
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="d20")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-roofline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--mfma-calibration", action="store_true")
    ap.add_argument("--optimizer", action="store_true",
                    help="time the optimiser step (Muon + AdamW) over the configuration's parameters")
    ap.add_argument("--decode", action="store_true",
                    help="time KV-cache inference: prefill of a 512-token prompt, then sampled decode steps")
    ap.add_argument("--decode-nseq", default="1,8,16", help="sequences per decode batch, comma-separated")
    ap.add_argument("--library-gemm", action="store_true",
                    help="time the vendor BLAS (torch.matmul) next to nc_op_matmul on the d20 product shapes")
    ap.add_argument("--cpu-sample-tokens", type=int, default=2048)
    return ap.parse_args()


def kernel_source_hash(family: str) -> str:
    src = "attn_mfma.h" if family.startswith("attn") else "gemm_mfma.h"
    csrc = os.path.join(ROOT, "decoder_only_transformer_d20_amd", "csrc")
    names = [src, "k_attn_mfma.hip"] if family.startswith("attn") else [src]
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(csrc, n), "rb").read())
    return h.hexdigest()[:16]


def to_dev(a, bf16):
    import numpy as np
    import torch
    import synthdata
    if bf16:
        return torch.from_numpy(synthdata.f32_to_bf16_bits(a).view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))


def mfma_loop_tflops(torch, nc, stream, iters=4000):
    """bf16 TFLOP/s of nc_op_mfma_loop with one block (4 waves) per CU."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sink = torch.empty(cus * 256, dtype=torch.float32, device="cuda")
    nc.ops.mfma_loop(iters, cus, sink, stream.cuda_stream)               # warm-up
    ev0.record(stream)
    nc.ops.mfma_loop(iters, cus, sink, stream.cuda_stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    return round(cus * 4 * iters * 8 * 32768 / (ev0.elapsed_time(ev1) * 1e-3) / 1e12, 1)


def wgrad_splits(M, N, K, cus=256):
    """The split-K count the library picks for a weight-gradient product:
    the count minimising (compute at 1 PFLOP/s x wave quantisation) + the
    fp32 partials' round trip at 5 TB/s, over 256 x 256 tiles."""
    tiles = (M // 256) * (N // 256)
    best_s, best = 1, None
    for s in range(1, min(32, K // 64) + 1):
        units = tiles * s
        waves = -(-units // cus)
        t = 2.0 * M * N * K / 1e15 * (waves * cus / units) + (s * 8.0 * M * N / 5e12 if s > 1 else 0.0)
        if best is None or t < best * (1.0 - 1e-9):
            best, best_s = t, s
    return best_s


def library_gemm(reps=10):
    """TFLOP/s of the vendor BLAS (torch.matmul, bf16 in and out) and of
    nc_op_matmul on the products of one d20 step (32 x 2048 tokens), same
    operands and transposition.  nc's weight-gradient products write fp32
    (split-K as in the step); the BLAS writes bf16, which only favours it.
    The step's own kernels also fuse epilogues (rotary, relu^2, residual,
    log-sum-exp) that these plain products leave out."""
    import torch
    import decoder_only_transformer_d20_amd as nc
    stream = torch.cuda.current_stream()
    T, d, F, V = 32 * 2048, 1280, 5120, 65536
    g = torch.Generator(device="cuda").manual_seed(0)
    rnd = lambda *shape: (torch.randn(*shape, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    # (name, M, N, K, p_trans, q_trans, out_f32) in C[m][n] = sum_k P[m][k] Q[n][k]
    shapes = [("fwd qkv", T, 3 * d, d, 0, 0, 0), ("fwd attn-out", T, d, d, 0, 0, 0),
              ("fwd mlp-up", T, F, d, 0, 0, 0), ("fwd mlp-down", T, d, F, 0, 0, 0),
              ("fwd head", T, V, d, 0, 0, 0),
              ("dgrad qkv", T, d, 3 * d, 0, 1, 0), ("dgrad mlp-up", T, d, F, 0, 1, 0),
              ("dgrad mlp-down", T, F, d, 0, 1, 0), ("dgrad head", T, d, V, 0, 1, 0),
              ("wgrad qkv", 3 * d, d, T, 1, 1, 1), ("wgrad attn-out", d, d, T, 1, 1, 1),
              ("wgrad mlp-up", F, d, T, 1, 1, 1), ("wgrad mlp-down", d, F, T, 1, 1, 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn):
        fn()
        ev[0].record(stream)
        for _ in range(reps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    rows = []
    for name, M, N, K, pt, qt, f32 in shapes:
        P = rnd(K, M) if pt else rnd(M, K)
        Q = rnd(K, N) if qt else rnd(N, K)
        s = wgrad_splits(M, N, K) if f32 else 1
        C = torch.empty(M, N, dtype=torch.float32 if f32 else torch.bfloat16, device="cuda")
        part = torch.empty(s * M * N if s > 1 else 1, dtype=torch.float32, device="cuda")
        Pm = P.t() if pt else P                   # [M][K] view
        Qm = Q if qt else Q.t()                   # [K][N] view
        ms_nc = timed(lambda: nc.ops.matmul(nc.DTYPE_BF16, pt, qt, M, N, K, P, Q, C, f32, s, part, 0,
                                            stream.cuda_stream))
        ms_lib = timed(lambda: torch.matmul(Pm, Qm))
        ref = torch.matmul(Pm, Qm).float()
        err = ((C.float() - ref).abs().max() / ref.abs().max()).item()
        fl = 2.0 * M * N * K
        rows.append({"product": name, "M": M, "N": N, "K": K, "splits": s,
                     "nc_tflops": round(fl / (ms_nc * 1e-3) / 1e12, 1),
                     "blas_tflops": round(fl / (ms_lib * 1e-3) / 1e12, 1),
                     "nc_over_blas": round(ms_lib / ms_nc, 3), "max_rel_diff": float(f"{err:.2e}")})
        print(f"[library-gemm] {rows[-1]}", file=sys.stderr, flush=True)
        del P, Q, C, part, ref
    blas = getattr(torch.backends.cuda, "preferred_blas_library", lambda: None)()
    print(json.dumps({"library_gemm": rows, "blas": str(blas), "reps": reps}), flush=True)


def optimizer_timing(torch, nc, cfg, steps=5, warmup=1, trace=True):
    """Time nc_optimizer_step over every parameter of cfg: fp32 master
    weights, bf16 model copy, seeded fp32 gradients, optimiser state from
    zero.  Returns ms per step and, per traced family, launches, ms and
    rate (Newton-Schulz products in TFLOP/s, AdamW in GB/s of its
    algorithmic 30 bytes per element)."""
    import numpy as np
    import synthdata
    c = nc.make_config(cfg)
    sess = nc.Session(cfg)
    stream = sess.stream
    P = synthdata.param_count(cfg)
    g = torch.Generator(device="cuda").manual_seed(7)
    master = (torch.randn(P, device="cuda", generator=g) * 0.02).float()
    grads = (torch.randn(P, device="cuda", generator=g) * 0.001).float()
    params = torch.empty(P, dtype=torch.bfloat16 if cfg.dtype == "bf16" else torch.float32, device="cuda")
    state = torch.zeros(nc.optim_state_bytes(c) // 4, dtype=torch.float32, device="cuda")
    scratch = torch.empty(nc.optim_scratch_bytes(c) + 256, dtype=torch.uint8, device="cuda")
    sp = (scratch.data_ptr() + 255) // 256 * 256
    h = nc.optim_default(c, 0, 1000, n_micro=8)

    def step():
        sess.optimizer_step(master, params, grads, state, sp, h)

    for _ in range(warmup):
        step()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(steps):
        step()
    ev[1].record(stream)
    torch.cuda.synchronize()
    out = {"ms_per_step": round(ev[0].elapsed_time(ev[1]) / steps, 3)}
    if trace:
        fam = {}
        for f in nc.OPTIM_TRACE_FAMILIES:
            sess.trace_enable(f)
            step()
            n, ms, fl, by = sess.trace_read()
            rate = {"tflops": round(fl / (ms * 1e-3) / 1e12, 1)} if fl else {"gbps": round(by / (ms * 1e-3) / 1e9, 1)}
            fam[f] = {"launches": n, "ms": round(ms, 3), **rate, "flops": fl, "bytes": by}
        sess.trace_enable(None)
        out["families"] = fam
    del master, grads, params, state, scratch
    return out


def decode_timing(torch, nc, cfg, nseqs=(1, 8, 16), prompt=512, steps=128):
    """Time nc_prefill + nc_decode + nc_sample on the configuration's model.
    Per batch of nseq sequences: one prefill of a `prompt`-token prompt,
    then `steps` decode steps, each followed by sampling (temperature 1,
    top-k 50, uniforms drawn beforehand on the device).  The decode rate
    is tokens/s over the timed steps; the HBM rate counts each step's
    algorithmic bytes: every block matrix and U once, nseq rows of E, the
    keys and values read so far, the new K/V and the fp32 logits."""
    import numpy as np
    import synthdata
    d, V, L, F = cfg.d_model, cfg.vocab, cfg.n_layer, cfg.d_ff
    es = 2 if cfg.dtype == "bf16" else 4
    pcfg = cfg.with_(batch=1, seq_len=prompt)
    c = nc.make_config(pcfg)
    sess = nc.Session(pcfg)
    stream = sess.stream
    params = synthdata.make_params(cfg)
    P = torch.from_numpy(synthdata.f32_to_bf16_bits(params).view(np.int16) if es == 2 else params).cuda()
    g = torch.Generator(device="cuda").manual_seed(11)
    idx = torch.randint(0, V, (prompt,), device="cuda", generator=g, dtype=torch.int32)
    res = []
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for nseq in nseqs:
        ml = prompt + steps + 1
        kv = torch.zeros(nc.kv_cache_bytes(c, nseq, ml), dtype=torch.uint8, device="cuda")
        scr = torch.empty(nc.decode_scratch_bytes(c, nseq, ml) + 256, dtype=torch.uint8, device="cuda")
        sp = (scr.data_ptr() + 255) // 256 * 256
        logits = torch.empty(nseq, V, dtype=torch.float32, device="cuda")
        u = torch.rand(steps + 1, nseq, device="cuda", generator=g)
        tok = torch.empty(steps + 1, nseq, dtype=torch.int32, device="cuda")
        sscr = torch.empty(nc.sample_scratch_bytes(nseq, V) + 256, dtype=torch.uint8, device="cuda")
        ssp = (sscr.data_ptr() + 255) // 256 * 256
        # warm-up pass (also the first run of every kernel)
        sess.prefill(P, idx, prompt, nseq, kv, nseq, ml, logits)
        sess.decode(P, idx[:nseq], nseq, prompt, kv, nseq, ml, sp, logits)
        torch.cuda.synchronize()
        ev[0].record(stream)
        sess.prefill(P, idx, prompt, nseq, kv, nseq, ml, logits)
        ev[1].record(stream)
        nc.sample_parallel(logits, 1, V, 1.0, 50, u[0], tok[0], ssp, stream.cuda_stream)
        if nseq > 1:
            tok[0].copy_(tok[0, :1].expand(nseq))
        ev[2].record(stream)
        for i in range(steps):
            sess.decode(P, tok[i], nseq, prompt + i, kv, nseq, ml, sp, logits)
            nc.sample_parallel(logits, nseq, V, 1.0, 50, u[i + 1], tok[i + 1], ssp, stream.cuda_stream)
        ev[3].record(stream)
        torch.cuda.synchronize()
        t_pre = ev[0].elapsed_time(ev[1])
        t_dec = ev[2].elapsed_time(ev[3]) / steps
        kv_read = sum(nseq * (prompt + i + 1) * 2 * d * L * es for i in range(steps)) / steps
        step_bytes = (12 * L * d * d + V * d) * es + nseq * d * es + kv_read + nseq * 2 * d * L * es + nseq * V * 4
        res.append({"nseq": nseq, "prompt_tokens": prompt, "decode_steps": steps,
                    "prefill_ms": round(t_pre, 3), "prefill_tokens_per_s": round(prompt / (t_pre * 1e-3), 1),
                    "decode_ms_per_step": round(t_dec, 4),
                    "decode_tokens_per_s": round(nseq / (t_dec * 1e-3), 1),
                    "decode_hbm_gbps": round(step_bytes / (t_dec * 1e-3) / 1e9, 1),
                    "decode_hbm_frac_of_8tbps": round(step_bytes / (t_dec * 1e-3) / 8e12, 4),
                    "decode_bytes_per_step": step_bytes})
        print(f"[decode] {res[-1]}", file=sys.stderr, flush=True)
        del kv, scr
    return res


def measured_peaks(torch, nc, stream):
    """What the chip sustains on this machine, next to the spec peaks: the bf16
    matrix-core rate of a register-only MFMA loop (nc_op_mfma_loop: 8
    independent 32x32x16 products per iteration, no memory traffic), and HBM
    read+write bandwidth of a 2 GiB device-to-device copy."""
    import ctypes
    props = torch.cuda.get_device_properties(0)
    info = [ctypes.c_int32() for _ in range(4)]
    nc.ops.device_info(torch.cuda.current_device(), *[ctypes.byref(x) for x in info])
    hip_cus, clock_khz, mem_clock_khz, bus_bits = (x.value for x in info)
    mfma_tflops = mfma_loop_tflops(torch, nc, stream)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 2 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    with torch.cuda.stream(stream):
        b.copy_(a)                                                        # warm-up
        ev0.record(stream)
        for _ in range(3):
            b.copy_(a)
        ev1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 3 * 2 * n / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del a, b
    # dense bf16 on CDNA4: 4096 FLOP per clock per CU, which gives the
    # 2.5 PFLOP/s figure at 256 CUs and 2.4 GHz
    return {"device": props.name, "compute_units": hip_cus, "peak_clock_mhz": clock_khz / 1000,
            "bf16_dense_peak_at_peak_clock_tflops": round(hip_cus * 4096 * clock_khz * 1e3 / 1e12, 1),
            "memory_clock_mhz": mem_clock_khz / 1000, "memory_bus_bits": bus_bits,
            "mfma_loop_tflops": mfma_tflops,
            "hbm_copy_gbps": round(copy_gbps, 1),
            "note": "mfma_loop: register-only bf16 MFMA loop on every CU; hbm_copy: read+write bytes of a "
                    "2 GiB device copy"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.library_gemm:
        library_gemm()
        return
    if args.decode:
        import torch
        import synthdata
        import decoder_only_transformer_d20_amd as nc
        cfg = synthdata.get_config(args.config)
        r = decode_timing(torch, nc, cfg, nseqs=tuple(int(x) for x in args.decode_nseq.split(",")))
        print(json.dumps({"metric": "KV-cache decode tokens/s (sampled, temperature 1, top-k 50)",
                          "config": {"workload": f"{cfg.name}: prefill of a 512-token prompt, then 128 decode "
                                                 f"steps per batch of sequences, {cfg.dtype}"},
                          "roofline": {"bound": "hbm", "peak": 8000.0, "unit": "GB/s",
                                       "achieved_by_nseq": {str(x["nseq"]): x["decode_hbm_gbps"] for x in r}},
                          "results": r}), flush=True)
        return
    if args.optimizer:
        import torch
        import synthdata
        import decoder_only_transformer_d20_amd as nc
        cfg = synthdata.get_config(args.config)
        r = optimizer_timing(torch, nc, cfg, steps=args.steps, warmup=args.warmup)
        ns = r["families"]["optim_ns"]
        print(json.dumps({"metric": "optimiser step time (Muon on every matrix, AdamW on E and U)",
                          "config": {"workload": f"{cfg.name}: {synthdata.param_count(cfg)} parameters, "
                                                 f"bf16 Newton-Schulz, fp32 master weights and state"},
                          "steps": args.steps, "warmup": args.warmup, **r,
                          "roofline": {"bound": "mfma", "kernel_family": "optim_ns",
                                       "achieved": ns["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                       "frac": round(ns["tflops"] / PEAK_BF16_TFLOPS, 4)}}), flush=True)
        return
    if args.mfma_calibration:
        import torch
        import decoder_only_transformer_d20_amd as nc
        print(json.dumps({"mfma_loop_tflops": mfma_loop_tflops(torch, nc, torch.cuda.current_stream())}))
        return
    import numpy as np
    import torch
    import synthdata
    import decoder_only_transformer_d20_amd as nc
    from decoder_only_transformer_d20_amd.flops import flops_per_step, flops_per_token, flops_per_token_causal

    cfg = synthdata.get_config(args.config)
    if cfg.block_only:
        block_bench(args, cfg)
        return
    bf16 = cfg.dtype == "bf16"
    N = cfg.batch * cfg.seq_len
    t0 = time.time()
    params = synthdata.make_params(cfg)
    idx, tgt = synthdata.make_tokens(cfg)
    tb = synthdata.make_token_bytes(cfg)
    print(f"[bench] inputs drawn in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    sess = nc.Session(cfg)
    stream = sess.stream
    P = to_dev(params, bf16)
    I, Tg, TB = to_dev(idx.ravel(), False), to_dev(tgt.ravel(), False), to_dev(tb, False)
    ce = torch.empty(N, dtype=torch.float32, device="cuda")
    out = torch.empty(5, dtype=torch.float64, device="cuda")
    G = torch.empty(params.size, dtype=torch.float32, device="cuda")

    def step():
        sess.forward(P, I, Tg, ce)
        sess.loss_bpb(TB, out)
        sess.backward(P, G)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    # per-family breakdown (untimed): one traced step per family
    families = {}
    dominant = None
    if not args.no_roofline:
        for f in nc.TRACE_FAMILIES:
            sess.trace_enable(f)
            step()
            n, ms, fl, by = sess.trace_read()
            if n:
                families[f] = {"launches": n, "ms": round(ms, 3), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                               "alg_gb_per_launch": round(by / n / 1e9, 4)}
        sess.trace_enable(None)
        single = [f for f in families if f in nc.SINGLE_KERNEL_FAMILIES]
        dominant = max(single, key=lambda f: families[f]["ms"]) if single else None
        if dominant:
            sess.trace_enable(dominant)

    # one event between consecutive steps (on the library's stream): the
    # mean over the K steps is ms_per_step; median and min come from the
    # per-step intervals
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    loss, bpb = out.cpu().numpy()[:2]
    grads_finite = bool(torch.isfinite(G).all().item())
    tok_s = N / (ms * 1e-3)
    mfu = flops_per_step(cfg) / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)
    mfu_causal = flops_per_token_causal(cfg) * N / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)
    print(f"[bench] {ms:.2f} ms/step, {tok_s:,.0f} tok/s, MFU {mfu:.3f}, loss {loss:.4f}, bpb {bpb:.4f}",
          file=sys.stderr, flush=True)

    result = {
        "metric": METRIC if cfg.name == "d20" else
                  f"train tokens/s + MFU (fwd+bwd) on 1 MI355X, {cfg.name} at {cfg.batch}x{cfg.seq_len} tok/step",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "ms_per_step_median": round(per_step[len(per_step) // 2] if len(per_step) % 2
                                    else 0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2]), 3),
        "ms_per_step_min": round(per_step[0], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Zipf(1.1) tokens, 1+Poisson(3.8) bytes per id, N(0,1/sqrt(fan_in)) weights)",
        "config": {
            "workload": f"{cfg.name} training step: forward + CE/bpb + backward, {cfg.n_layer} layers x "
                        f"d{cfg.d_model}, {cfg.n_head}x{cfg.head_dim} heads, MLP {cfg.d_ff}, vocab {cfg.vocab}",
            "global_batch": cfg.batch,
            "seq_len": cfg.seq_len,
            "tokens_per_step": N,
            "parallelism": "none (1 GPU)",
        },
        "mfu": round(mfu, 4),
        "mfu_causal_attention": round(mfu_causal, 4),
        "model_flops_per_token": flops_per_token(cfg),
        "loss_nats": float(loss),
        "bpb": float(bpb),
        "grads_finite": grads_finite,
    }

    if dominant:
        n, tms, fl, by = sess.trace_read()
        sess.trace_enable(None)
        avg = tms / n * 1e-3
        achieved = fl / n / avg / 1e12
        tr = TRAFFIC.get(dominant)
        traffic = tr["bytes_per_launch"] if tr and tr["source_hash"] == kernel_source_hash(dominant) else None
        result["roofline"] = {
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel_family": dominant,
            "launches_timed": n,
            "avg_launch_ms": round(tms / n, 4),
            "flops_per_launch": fl / n,
            "algorithmic_bytes_per_launch": by / n,
            "kernel_source_hash": kernel_source_hash(dominant),
        }
        result["kernel_families"] = families
    del P, G
    if not args.no_roofline and not cfg.block_only:
        o = optimizer_timing(torch, nc, cfg, steps=3, warmup=1, trace=False)
        result["optimizer_step"] = {
            "ms": o["ms_per_step"],
            "note": "one Muon + AdamW step over every parameter, timed separately and not part of value; "
                    "the pages' batch of 2^19 tokens is 8 of these fwd+bwd steps per optimiser step"}
    if not args.no_roofline:
        result["measured_peaks"] = measured_peaks(torch, nc, stream)
        if "roofline" in result:
            result["roofline"]["frac_of_measured_mfma"] = round(
                result["roofline"]["achieved"] / result["measured_peaks"]["mfma_loop_tflops"], 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, params, idx, tgt, tb, args.cpu_sample_tokens)
    print(json.dumps(result), flush=True)


def block_bench(args, cfg):
    """One d20 layer at its real shape (32 x 2048 tokens, bf16): forward +
    backward of the block (nc_block_forward + nc_block_backward) per step,
    seeded N(0,1) input activations and upstream gradients."""
    import numpy as np
    import torch
    import synthdata
    import decoder_only_transformer_d20_amd as nc
    from decoder_only_transformer_d20_amd.flops import flops_per_step
    N = cfg.batch * cfg.seq_len
    params = synthdata.make_params(cfg)
    x, dy = synthdata.make_block_io(cfg)
    sess = nc.Session(cfg)
    stream = sess.stream
    P, X, DY = to_dev(params, True), to_dev(x.reshape(N, -1), True), to_dev(dy.reshape(N, -1), True)
    Y, DX = torch.empty_like(X), torch.empty_like(X)
    G = torch.empty(params.size, dtype=torch.float32, device="cuda")

    def step():
        sess.block_forward(P, X, Y)
        sess.block_backward(P, DY, DX, G)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    families = {}
    for f in nc.TRACE_FAMILIES:
        sess.trace_enable(f)
        step()
        n, ms, fl, by = sess.trace_read()
        if n:
            families[f] = {"launches": n, "ms": round(ms, 3), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                           "alg_gb_per_launch": round(by / n / 1e9, 4)}
    sess.trace_enable(None)
    single = [f for f in families if f in nc.SINGLE_KERNEL_FAMILIES]
    dominant = max(single, key=lambda f: families[f]["ms"])
    sess.trace_enable(dominant)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    n, tms, fl, by = sess.trace_read()
    sess.trace_enable(None)
    achieved = fl / n / (tms / n * 1e-3) / 1e12
    mfu = flops_per_step(cfg) / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)
    print(f"[bench] block: {ms:.3f} ms/step, MFU {mfu:.3f}", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = block_cpu_baseline(cfg, params, x, dy, args.cpu_sample_tokens)
        print(f"[bench] cpu baseline: {cpu['value']} tok/s on {cpu['cores']} cores", file=sys.stderr, flush=True)
    out = {
        "metric": "train tokens/s + MFU (fwd+bwd) of one d20 block on 1 MI355X, 32x2048 tok/step",
        "value": round(N / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "ms_per_step_min": round(per_step[0], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) activations and upstream gradients, N(0,1/sqrt(fan_in)) weights)",
        "config": {"workload": f"one d20 block: d{cfg.d_model}, {cfg.n_head}x{cfg.head_dim} heads, MLP {cfg.d_ff}, "
                               f"forward + backward", "global_batch": cfg.batch, "seq_len": cfg.seq_len,
                   "tokens_per_step": N, "parallelism": "none (1 GPU)"},
        "mfu": round(mfu, 4), "model_flops_per_step": flops_per_step(cfg),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None, "kernel_family": dominant,
                     "launches_timed": n, "avg_launch_ms": round(tms / n, 4), "flops_per_launch": fl / n},
        "kernel_families": families}
    if cpu:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


def block_cpu_baseline(cfg, params, x, dy, sample_tokens):
    """The fp64 oracle's block step (forward + backward of one layer, as
    written) on the first `sample_tokens` tokens of row 0."""
    import synthdata
    import oracle
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    T = min(sample_tokens, cfg.seq_len)
    c = cfg.with_(batch=1, seq_len=T)
    lp = synthdata.split_params(cfg, params)["layers"][0]
    t0 = time.time()
    oracle.block_step(c, lp, x[:1, :T].astype("float64"), dy[:1, :T].astype("float64"))
    dt = time.time() - t0
    return {"value": round(T / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 numpy oracle block step (fwd+bwd of one layer) on the first {T} tokens of row 0 "
                      f"of the {cfg.name} workload ({dt:.1f} s wall)"}


def cpu_baseline(cfg, params, idx, tgt, tb, sample_tokens):
    """The fp64 oracle (as written, untuned) on the first `sample_tokens`
    tokens of row 0: forward + loss + backward of that causal prefix.  Rows
    are independent and a prefix's losses equal the full row's at those
    positions, so this is a bounded slice of the same workload; per-token
    attention work grows with position, so a prefix slightly flatters the
    oracle against full 2048-token rows."""
    import synthdata
    import oracle
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    T = min(sample_tokens, cfg.seq_len)
    c = cfg.with_(batch=1, seq_len=T)
    p = synthdata.split_params(cfg, params)
    t0 = time.time()
    oracle.train_step(c, p, idx[:1, :T], tgt[:1, :T], tb)
    dt = time.time() - t0
    return {
        "value": round(T / dt, 3),
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"fp64 numpy oracle fwd+loss+bwd on the first {T} tokens of row 0 of the {cfg.name} "
                  f"workload ({dt:.1f} s wall)",
    }


if __name__ == "__main__":
    main()
