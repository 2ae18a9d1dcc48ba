"""Benchmark: one d20 training step (forward + loss/bpb + backward) per step on
one MI355X, through the C ABI (include/nc.h).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config d20]
                    [--no-cpu-baseline] [--no-roofline]

Prints one JSON line.  `value` is training tokens/s of the whole job with
inputs already resident in HBM; MFU uses the FLOP convention of
decoder_only_transformer_d20_amd.flops against the bf16 dense MFMA peak.
`roofline` reports the dominant kernel (the unembedding + log-sum-exp GEMM)
timed live with HIP events on its own stream; `cpu_baseline` times the fp64
oracle on a bounded prefix of one row on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "train tokens/s + MFU (fwd+bwd) on 1 MI355X, d20 at 32x2048 tok/step"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, TFLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="d20")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-roofline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=256)
    return ap.parse_args()


def to_dev(a, bf16):
    import numpy as np
    import torch
    import synthdata
    if bf16:
        return torch.from_numpy(synthdata.f32_to_bf16_bits(a).view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import synthdata
    import decoder_only_transformer_d20_amd as nc
    from decoder_only_transformer_d20_amd.flops import flops_per_step, flops_per_token, flops_per_token_causal

    cfg = synthdata.get_config(args.config)
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
    del params

    def step():
        sess.forward(P, I, Tg, ce)
        sess.loss_bpb(TB, out)
        sess.backward(P, G)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    loss, bpb = out.cpu().numpy()[:2]
    grads_finite = bool(torch.isfinite(G).all().item())
    tok_s = N / (ms * 1e-3)
    mfu = flops_per_step(cfg) / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)
    mfu_causal = flops_per_token_causal(cfg) * N / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)
    print(f"[bench] {ms:.2f} ms/step, {tok_s:,.0f} tok/s, MFU {mfu:.3f}, loss {loss:.4f}, bpb {bpb:.4f}",
          file=sys.stderr, flush=True)

    result = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
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

    if not args.no_roofline and not cfg.block_only:
        result["roofline"] = roofline_head(cfg, sess, P, Tg, nc, torch)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_sample_tokens)
    print(json.dumps(result), flush=True)


def roofline_head(cfg, sess, P, Tg, nc, torch):
    """Dominant kernel: the unembedding GEMM with the fused log-sum-exp
    epilogue (k_gemm_mfma<256,256,...,EPI_LSE>), launched alone at the
    step's shape through nc_op_head_gemm_lse and timed with HIP events on the
    stream it runs on.  Algorithmic work per launch = 2 * (B*T) * V * d."""
    N, d, V = cfg.batch * cfg.seq_len, cfg.d_model, cfg.vocab
    xf = torch.randn(N * d, device="cuda").to(torch.bfloat16).view(torch.int16)
    U_off, _, _ = nc.param_offset(cfg, "U")
    U = P[U_off:U_off + V * d]
    scratch = torch.empty(nc.ops.head_scratch_bytes(1, N, d, V, 0) // 4 + 64, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    for _ in range(2):
        nc.ops.head_gemm_lse(1, N, d, V, xf, U, Tg, scratch, s.cuda_stream)
    iters = 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(iters):
        nc.ops.head_gemm_lse(1, N, d, V, xf, U, Tg, scratch, s.cuda_stream)
    e1.record(s)
    torch.cuda.synchronize()
    dur = e0.elapsed_time(e1) / iters * 1e-3
    flops = 2.0 * N * V * d
    achieved = flops / dur / 1e12
    return {
        "kernel": "k_gemm_mfma<256,256,...,EPI_LSE> (unembedding GEMM + log-sum-exp partials)",
        "bound": "mfma",
        "achieved": round(achieved, 1),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": None,
        "launch_ms": round(dur * 1e3, 4),
        "flops_per_launch": flops,
    }


def cpu_baseline(cfg, sample_tokens):
    """The fp64 oracle (untuned) on the first `sample_tokens` tokens of row 0:
    forward + loss + backward of that causal prefix.  Rows are independent and
    the prefix's losses equal the full row's at those positions, so this is a
    bounded slice of the same workload; per-token attention work grows with
    the prefix length, so it slightly flatters the oracle against full rows."""
    import numpy as np
    import synthdata
    import oracle
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    params = synthdata.make_params(cfg)
    idx, tgt = synthdata.make_tokens(cfg, rows=1)
    tb = synthdata.make_token_bytes(cfg)
    T = min(sample_tokens, cfg.seq_len)
    c = cfg.with_(batch=1, seq_len=T)
    p = synthdata.split_params(cfg, params)
    t0 = time.time()
    oracle.train_step(c, p, idx[:, :T], tgt[:, :T], tb)
    dt = time.time() - t0
    return {
        "value": round(T / dt, 3),
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"fp64 numpy oracle fwd+loss+bwd on the first {T} tokens of row 0 of the {cfg.name} "
                  f"workload ({dt:.1f} s)",
    }


if __name__ == "__main__":
    main()
