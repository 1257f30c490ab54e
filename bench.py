#!/usr/bin/env python3
"""Benchmark of the joint-attention forward on one MI355X.

One step = one pass of the bf16 hot path over the 2048x2048 T2I step shape
(B=1, 24 heads x 128, 512 text + 128x128 image tokens = 16896 tokens): build
the 2D-axial RoPE table from the token positions, the K/V preparation (K
rotated, V transposed), then the attention forward with RoPE fused into the
Q load.  Inputs are seeded synthetic tensors resident in HBM before
the timed region.  Throughput is 4*B*H*S^2*D flops per step (QK^T + PV).

Also reported on the same JSON line:
  roofline      the attention forward's own average duration (HIP events on
                the launch stream, the K/V preparation excluded and reported
                beside it) against the bf16 dense MFMA peak;
  fp8           the FP8 path (RoPE+quantize pass, K/V preparation, FP8
                forward) timed the same way, against the fp8 MFMA peak and
                HBM bandwidth, and with the
                repair of the tokens with the largest quantization error
                (budget 0.005);
  qk_norm       the same passes with query/key RMS normalization fused
                where RoPE is (seeded weights): K/V preparation, forward,
                FP8 quantize;
  sparse        the block-sparse forwards (bf16, and FP8 on the FP8 leg's
                codes) on a seeded mask over 128-query x 64-key blocks at the
                block density of the sparse steps (half the blocks kept),
                against the flops of the kept blocks;
  gemm_context  a large bf16 GEMM through torch.matmul (the vendor BLAS) timed
                in the same run: the dense MFMA rate this power-limited part
                sustains in practice, next to which the forward's rate reads;
  cpu_baseline  the fp64 oracle timed on this host's cores over a bounded
                sample of query rows (scaled to TFLOP/s), plus the parity of
                the GPU output on those rows.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "joint-attention fwd TFLOP/s and % of MFMA peak at 2048x2048 (16896 tok)"
PEAK_BF16_TFLOPS = 2516.6    # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_FP8_TFLOPS = 5033.2     # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
REPAIR_BUDGET = 0.005        # the pages' vc_repair_budget
CSRC = os.path.join(ROOT, "joint_attention_attn_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def _log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the first launches run while the GPU clock ramps up (see profiles/)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="t2i_2048")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-sparse", action="store_true")
    ap.add_argument("--no-norm", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm-context", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain elementwise kernel that reads and writes BYTES "
                         "(fp32 negation), to calibrate HBM byte counters, then exit")
    return ap.parse_args()


def _traffic_for_current_kernel(kernel: str, workload: str, source: str):
    """HBM bytes per launch from a committed rocprofv3 counter record
    (profiles/<kernel>_<workload>_traffic.txt), only if it was taken on this
    workload and on the kernel source as it is now; None otherwise."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                key, val = line.split(":", 1)
                rec[key.strip()] = val.strip()
    with open(os.path.join(CSRC, source), "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if rec.get("source_sha256") != sha or "hbm_bytes_per_launch" not in rec:
        return None
    return float(rec["hbm_bytes_per_launch"])


def _time_launches(fn, n, short=False):
    """Run fn() n times with a HIP event pair around each launch on the
    current (launch) stream; returns per-launch ms.  short: the kernel takes
    less time than the host spends per call, so a bounded spin kernel first
    holds the stream for about 3 ms and the host has enqueued the timed
    launches before the GPU reaches them; a pair then brackets GPU time
    only.  (Millisecond kernels keep the host ahead by themselves.)"""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    if short:
        torch.cuda.synchronize()
        torch.cuda._sleep(6_000_000)    # clock cycles (~3 ms)
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def main() -> int:
    args = _parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the single-GPU joint-attention kernel; runs on more than "
              "one GPU are not part of this build (use --gpus 1).", file=sys.stderr)
        return 2

    import torch
    import joint_attention_attn_amd as ja
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = "cuda:0"
    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "bytes_written": 4 * n}))
        return 0
    w = synth.WORKLOADS[args.config]
    B, S, H, D = w.shape
    flops = w.flops()
    _log(f"[bench] workload {w.name}: B={B} S={S} H={H} D={D}, {flops / 1e12:.4f} TFLOP/step")

    q, k, v, outl = synth.make_qkv(w, args.seed)
    pos = synth.positions(w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    pos_d = torch.from_numpy(pos).to(dev)
    out = torch.empty_like(qd)
    torch.cuda.synchronize()

    def step():
        # the whole path in one call: RoPE table from the positions, K/V
        # preparation (K rotated, V transposed), forward (RoPE fused into the
        # Q load)
        ja.fwd_bf16(qd, kd, vd, pos_d, w.theta, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    _log(f"[bench] warmup {args.warmup} done")

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    _log(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step, {value:.1f} TFLOP/s")

    # dominant kernel: the attention forward (RoPE fused into the Q load),
    # timed per launch on K/V prepared once from the positions (prepared K/V,
    # RoPE table and coordinate table in one buffer, as the one-call path
    # builds them); the preparation kernel beside it, on a prebuilt table
    rope = ja.rope_table_2d(pos_d, D, w.theta)
    kv_pos = ja.prep_kv_bf16(kd, vd, pos_d, w.theta)
    n_t = max(args.steps, 5)
    kms = _time_launches(lambda: ja.fwd_bf16_prepared(qd, kv_pos, pos_d, w.theta, out=out), n_t)
    k_avg = sum(kms) / len(kms)
    pms = _time_launches(lambda: ja.prep_kv_bf16(kd, vd, rope=rope), n_t, short=True)
    prep_avg = sum(pms) / len(pms)
    tms = _time_launches(lambda: ja.rope_table_2d(pos_d, D, w.theta), n_t, short=True)
    table_avg = sum(tms) / len(tms)
    # the benchmarked output comes from the one-call path
    ja.fwd_bf16(qd, kd, vd, pos_d, w.theta, out=out)
    # algorithmic bytes of the preparation: read K, V and the table (fp64
    # cos, sin per pair), write both
    prep_bytes = 4 * B * S * H * D * 2 + S * (D // 2) * 16
    achieved = flops / (k_avg * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": _traffic_for_current_kernel("attn_fwd_bf16", w.name, "attn_bf16.hip"),
                "kernel": "attn_fwd_bf16_kernel<128, true, false, false> (+ merge_split_kernel of the "
                          "split last round); K/V preparation in prep_kv",
                "kernel_ms": round(k_avg, 4), "kernel_ms_min": round(min(kms), 4),
                "kernel_ms_median": round(sorted(kms)[len(kms) // 2], 4),
                "rope_table_ms": round(table_avg, 4),
                "prep_kv": {"ms": round(prep_avg, 4),
                            "traffic": _traffic_for_current_kernel("prep_kv_bf16", w.name, "prep_kv.hip"),
                            "gbs": round(prep_bytes / (prep_avg * 1e-3) / 1e9, 1),
                            "frac_of_hbm": round(prep_bytes / (prep_avg * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                                 4)}}
    _log(f"[bench] fwd kernel avg {k_avg:.3f} ms -> {achieved:.1f} TFLOP/s "
         f"({100 * achieved / PEAK_BF16_TFLOPS:.1f}% of bf16 peak); K/V prep {prep_avg:.3f} ms, "
         f"table {table_avg:.3f} ms")

    gemm = None if args.no_gemm_context else _gemm_context(achieved, max(args.steps, 5))

    fp8 = None
    fp8_outs = None
    if not args.no_fp8:
        q8, k8, v8, sq, sk, sv = ja.quant_rope_fp8(qd, kd, vd, rope=rope)
        kv8 = ja.prep_kv_fp8(k8, v8, sk, sv)
        out8 = torch.empty_like(out)
        for _ in range(2):
            ja.quant_rope_fp8(qd, kd, vd, rope=rope)
            ja.prep_kv_fp8(k8, v8, sk, sv)
            ja.fwd_fp8_prepared(q8, sq, kv8, out=out8)
        torch.cuda.synchronize()
        n = max(args.steps, 5)
        qms = _time_launches(lambda: ja.quant_rope_fp8(qd, kd, vd, rope=rope), n, short=True)
        pp8 = _time_launches(lambda: ja.prep_kv_fp8(k8, v8, sk, sv), n, short=True)
        fms = _time_launches(lambda: ja.fwd_fp8_prepared(q8, sq, kv8, out=out8), n)
        q_avg, pp_avg, f_avg = sum(qms) / n, sum(pp8) / n, sum(fms) / n
        elems = B * S * H * D
        q_bytes = 3 * elems * 2 + S * (D // 2) * 16 + 3 * elems + 3 * B * H * S * 4
        # preparation: read K and V codes and two scales, write the prepared
        # K, V^T and 16 bytes of per-key values per key (64-key padding aside)
        pp_bytes = 2 * elems + 2 * B * H * S * 4 + 2 * elems + B * H * S * 16
        f_tf = flops / (f_avg * 1e-3) / 1e12
        fp8 = {"fwd_ms": round(f_avg, 4), "fwd_tflops": round(f_tf, 2),
               "fwd_frac_of_fp8_peak": round(f_tf / PEAK_FP8_TFLOPS, 4),
               "fwd_traffic": _traffic_for_current_kernel("attn_fwd_fp8", w.name, "attn_fp8.hip"),
               "quant_ms": round(q_avg, 4),
               "quant_gbs": round(q_bytes / (q_avg * 1e-3) / 1e9, 1),
               "quant_frac_of_hbm": round(q_bytes / (q_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
               "quant_traffic": _traffic_for_current_kernel("quant_rope_fp8", w.name, "quant_fp8.hip"),
               "prep_ms": round(pp_avg, 4),
               "prep_gbs": round(pp_bytes / (pp_avg * 1e-3) / 1e9, 1),
               "prep_frac_of_hbm": round(pp_bytes / (pp_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
               "prep_traffic": _traffic_for_current_kernel("prep_kv_fp8", w.name, "prep_kv_fp8.hip"),
               "path_tflops": round(flops / ((f_avg + q_avg + pp_avg) * 1e-3) / 1e12, 2)}
        _log(f"[bench] fp8: fwd {f_avg:.3f} ms ({f_tf:.1f} TFLOP/s), quant {q_avg:.3f} ms "
             f"({fp8['quant_gbs']} GB/s), K/V prep {pp_avg:.3f} ms ({fp8['prep_gbs']} GB/s)")
        # repair of the tokens with the largest quantization error, at the
        # pages' budget 0.005
        n_rep = ja.repair_count(REPAIR_BUDGET, S)
        rp = ja.fp8_repair_plan(kd, vd, k8, v8, sk, sv, n_rep, rope=rope)
        kv8r = ja.prep_kv_fp8(k8, v8, sk, sv, repair=rp)
        out8r = torch.empty_like(out)
        for _ in range(2):
            ja.fwd_fp8_prepared(q8, sq, kv8r, out=out8r, repair=rp)
        torch.cuda.synchronize()
        pms = _time_launches(lambda: ja.fp8_repair_plan(kd, vd, k8, v8, sk, sv, n_rep, rope=rope),
                             n, short=True)
        rms = _time_launches(lambda: ja.fwd_fp8_prepared(q8, sq, kv8r, out=out8r, repair=rp), n)
        p_avg, r_avg = sum(pms) / n, sum(rms) / n
        fp8["repair"] = {"budget": REPAIR_BUDGET, "tokens_per_head": n_rep,
                         "plan_ms": round(p_avg, 4), "fwd_ms": round(r_avg, 4),
                         "fwd_tflops": round(flops / (r_avg * 1e-3) / 1e12, 2),
                         "path_tflops": round(flops / ((q_avg + p_avg + pp_avg + r_avg) * 1e-3)
                                              / 1e12, 2)}
        _log(f"[bench] fp8 + repair ({n_rep} tokens/head): plan {p_avg:.3f} ms, fwd {r_avg:.3f} ms")
        fp8_outs = (out8, out8r)

    qk_norm = None
    if not args.no_norm:
        qk_norm = _norm_leg(ja, w, qd, kd, vd, rope, pos_d, out, k_avg, prep_avg,
                            fp8["quant_ms"] if fp8 else None, max(args.steps, 5), args.seed)

    sparse = None
    if not args.no_sparse:
        fp8_in = (q8, sq, kv8, fp8["fwd_ms"]) if fp8 else None
        sparse = _sparse_leg(ja, w, qd, kv_pos, pos_d, out, k_avg, max(args.steps, 5), args.seed,
                             fp8_in)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = _cpu_baseline(w, q, k, v, pos, outl, out, args.cpu_seconds, fp8_outs)

    rec = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"{w.name}: joint text+image attention fwd, "
                                  f"{w.n_text} text + {w.grid}x{w.grid} image tokens"
                                  + (f" + {w.n_ref} reference grid(s)" if w.n_ref else "")
                                  + ", 2D-axial RoPE, N(0,1) bf16 with "
                                  f"{100 * w.outlier_frac:g}% x{w.outlier_scale:g} outlier tokens",
                      "batch": B, "seq_len": S, "heads": H, "head_dim": D,
                      "flops_per_step": flops},
           "roofline": roofline, "gemm_context": gemm, "cpu_baseline": cpu, "fp8": fp8,
           "qk_norm": qk_norm,
           "sparse": sparse}
    print(json.dumps(rec), flush=True)
    return 0


def _gemm_context(fwd_tflops, n):
    """A 16384 x 16384 x 8192 bf16 GEMM through torch.matmul, timed per
    launch like the forward: the practical dense bf16 MFMA rate of this GPU
    under its power limit, for context (not part of the hot path)."""
    import torch
    m, nn, kk = 16384, 16384, 8192
    g = torch.Generator(device="cpu").manual_seed(1234)
    a = torch.randn(m, kk, generator=g).to(device="cuda:0", dtype=torch.bfloat16)
    b = torch.randn(kk, nn, generator=g).to(device="cuda:0", dtype=torch.bfloat16)
    c = torch.empty(m, nn, device="cuda:0", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    ms = _time_launches(lambda: torch.matmul(a, b, out=c), n)
    avg = sum(ms) / len(ms)
    tf = 2.0 * m * nn * kk / (avg * 1e-3) / 1e12
    _log(f"[bench] torch.matmul bf16 {m}x{nn}x{kk}: {avg:.3f} ms, {tf:.1f} TFLOP/s")
    del a, b, c
    return {"op": f"torch.matmul bf16 {m}x{nn}x{kk}", "ms": round(avg, 4),
            "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "fwd_over_gemm": round(fwd_tflops / tf, 4)}


def _norm_leg(ja, w, qd, kd, vd, rope, pos_d, out, fwd_ms, prep_ms, quant_ms, n, seed):
    """Query/key RMS normalization fused into the passes that apply RoPE:
    their times with it, beside the times without (same run)."""
    import torch
    import synth
    B, S, H, D = w.shape
    gq, gk = (torch.from_numpy(g).to(qd.device) for g in synth.make_norm_weights(D, seed))
    kv = ja.prep_kv_bf16(kd, vd, pos_d, w.theta, k_norm=gk)
    # its own output buffer: `out` keeps the plain forward's result, which
    # the CPU baseline checks
    outn = torch.empty_like(out)
    for _ in range(3):
        ja.fwd_bf16_prepared(qd, kv, pos_d, w.theta, out=outn, q_norm=gq)
    torch.cuda.synchronize()
    pm = _time_launches(lambda: ja.prep_kv_bf16(kd, vd, rope=rope, k_norm=gk), n, short=True)
    fm = _time_launches(lambda: ja.fwd_bf16_prepared(qd, kv, pos_d, w.theta, out=outn, q_norm=gq),
                        n)
    p_avg, f_avg = sum(pm) / n, sum(fm) / n
    rec = {"weights": "seeded g = 1 + 0.1 N(0,1), eps 1e-6",
           "prep_kv_ms": round(p_avg, 4), "prep_kv_ms_without": round(prep_ms, 4),
           "fwd_ms": round(f_avg, 4), "fwd_ms_without": round(fwd_ms, 4)}
    if quant_ms is not None:
        qm = _time_launches(lambda: ja.quant_rope_fp8(qd, kd, vd, rope=rope, q_norm=gq, k_norm=gk),
                            n, short=True)
        rec["quant_ms"] = round(sum(qm) / n, 4)
        rec["quant_ms_without"] = round(quant_ms, 4)
    _log(f"[bench] qk norm: prep {p_avg:.3f} ms (without {prep_ms:.3f}), fwd {f_avg:.3f} ms "
         f"(without {fwd_ms:.3f})" + (f", quant {rec['quant_ms']:.3f} ms (without {quant_ms:.3f})"
                                     if quant_ms is not None else ""))
    return rec


def _sparse_leg(ja, w, qd, kv, pos_d, out, dense_ms, n, seed, fp8_in=None):
    """Block-sparse forwards on the seeded mask of the workload: kernel time,
    the flops of the kept blocks per second, and the fraction of the key
    blocks staged (a workgroup covers one query block and stages the key
    blocks it keeps); bf16, and FP8 on the FP8 leg's prepared K/V."""
    import numpy as np
    import torch
    import synth
    B, S, H, D = w.shape
    mask = synth.make_block_mask(w, synth.SPARSE_DENSITY, seed)
    m = mask.numpy().astype(bool)
    qb, kb = ja.SPARSE_QUERY_BLOCK, ja.SPARSE_KEY_BLOCK
    qrows = np.minimum(S - qb * np.arange(m.shape[2]), qb)
    kcols = np.minimum(S - kb * np.arange(m.shape[3]), kb)
    pairs = float((m * qrows[:, None] * kcols[None, :]).sum())
    kept_flops = 4.0 * D * pairs
    staged = m.mean()
    mask_d = mask.to(qd.device)
    outs = torch.empty_like(out)
    for _ in range(3):
        ja.fwd_bf16_block_sparse_prepared(qd, kv, mask_d, pos_d, w.theta, out=outs)
    torch.cuda.synchronize()
    ms = _time_launches(lambda: ja.fwd_bf16_block_sparse_prepared(qd, kv, mask_d, pos_d, w.theta,
                                                                  out=outs), n)
    avg = sum(ms) / n
    tf = kept_flops / (avg * 1e-3) / 1e12
    _log(f"[bench] sparse (density {synth.SPARSE_DENSITY}): {avg:.3f} ms, {tf:.1f} TFLOP/s of "
         f"kept blocks, {dense_ms / avg:.2f}x the dense kernel")
    rec = {"mask": f"seeded iid blocks of {qb}x{kb}, kept with p={synth.SPARSE_DENSITY}",
           "kept_frac": round(float(m.mean()), 4), "staged_frac": round(float(staged), 4),
           "kept_flops": kept_flops, "fwd_ms": round(avg, 4), "fwd_tflops": round(tf, 2),
           "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
           "speedup_vs_dense_kernel": round(dense_ms / avg, 3)}
    if fp8_in is not None:
        q8, sq, kv8, fp8_dense_ms = fp8_in
        for _ in range(3):
            ja.fwd_fp8_block_sparse_prepared(q8, sq, kv8, mask_d, out=outs)
        torch.cuda.synchronize()
        ms8 = _time_launches(lambda: ja.fwd_fp8_block_sparse_prepared(q8, sq, kv8, mask_d,
                                                                      out=outs), n)
        avg8 = sum(ms8) / n
        tf8 = kept_flops / (avg8 * 1e-3) / 1e12
        _log(f"[bench] fp8 sparse: {avg8:.3f} ms, {tf8:.1f} TFLOP/s of kept blocks, "
             f"{fp8_dense_ms / avg8:.2f}x the dense fp8 kernel")
        rec["fp8"] = {"fwd_ms": round(avg8, 4), "fwd_tflops": round(tf8, 2),
                      "frac_of_fp8_peak": round(tf8 / PEAK_FP8_TFLOPS, 4),
                      "speedup_vs_dense_fp8_kernel": round(fp8_dense_ms / avg8, 3)}
    return rec


def _cpu_baseline(w, q, k, v, pos, outl, out_gpu, target_s, fp8_outs=None):
    """The fp64 oracle on this host's cores over a bounded sample of query
    rows (all keys, all heads), scaled to TFLOP/s; plus the parity of the GPU
    output on those rows, the distance of the FP8 and repaired FP8 outputs
    from the bf16 path's oracle on them, and the FP8 output's parity with the
    oracle's own FP8 path (its quantizer, then fp64 attention on the
    dequantized codes) on the first rows of the sample."""
    import numpy as np
    import torch
    import oracle

    threads = torch.get_num_threads()
    cores = len(os.sched_getaffinity(0))
    B, S, H, D = w.shape
    rng = np.random.default_rng(7)
    order = rng.permutation(S)
    done_rows, spent, chunk = [], 0.0, 64
    got_all = out_gpu.cpu()
    f8_all = [t.cpu() for t in fp8_outs] if fp8_outs else []
    f8_num = [0.0] * len(f8_all)
    errs_num, errs_den = 0.0, 0.0
    while spent < target_s and len(done_rows) < S:
        rows = np.sort(order[len(done_rows):len(done_rows) + chunk])
        t0 = time.perf_counter()
        ref, _ = oracle.joint_attention(q, k, v, pos, w.theta, rows=rows)
        spent += time.perf_counter() - t0
        got = got_all[:, rows].double()
        errs_num += float(((got - ref) ** 2).sum())
        errs_den += float((ref ** 2).sum())
        for i, t in enumerate(f8_all):
            f8_num[i] += float(((t[:, rows].double() - ref) ** 2).sum())
        done_rows.extend(rows.tolist())
        chunk = min(chunk * 2, 1024)
    n = len(done_rows)
    sample_flops = 4.0 * B * H * n * S * D
    tflops = sample_flops / spent / 1e12
    _log(f"[bench] cpu oracle: {n} query rows x {H} heads in {spent:.1f} s on {threads} "
         f"threads ({cores} cores in the affinity mask) -> {tflops * 1e3:.2f} GFLOP/s")
    rec = {"value": round(tflops, 6), "unit": "TFLOP/s", "cores": cores, "torch_threads": threads,
           "kind": "oracle",
           "sample": f"{n} random query rows x {B * H} (batch, head) pairs x all {S} keys "
                     f"({sample_flops / 1e9:.1f} GFLOP) of {w.name}, fp64 torch-CPU",
           "seconds": round(spent, 2),
           "gpu_rel_l2_on_sample": round(math.sqrt(errs_num / errs_den), 6)}
    if f8_all:
        rec["fp8_vs_bf16_oracle_rel_l2_on_sample"] = round(math.sqrt(f8_num[0] / errs_den), 6)
        rec["fp8_repair_vs_bf16_oracle_rel_l2_on_sample"] = round(math.sqrt(f8_num[1] / errs_den), 6)
        # the FP8 criterion: the oracle run on its own dequantized codes
        rows = np.sort(order[:256])
        t0 = time.perf_counter()
        codes = oracle.quant_rope_fp8(q, k, v, pos, w.theta)
        ref8, _ = oracle.fp8_attention(*codes, rows=rows)
        got8 = f8_all[0][:, rows].double()
        rec["fp8_rel_l2_vs_fp8_oracle"] = round(float((got8 - ref8).norm() / ref8.norm()), 6)
        rec["fp8_oracle_rows"] = len(rows)
        _log(f"[bench] fp8 vs the oracle's FP8 path on {len(rows)} rows: "
             f"rel-L2 {rec['fp8_rel_l2_vs_fp8_oracle']:.3e} ({time.perf_counter() - t0:.1f} s)")
    return rec


if __name__ == "__main__":
    sys.exit(main())
