"""Benchmark of the sliding-window paged attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input that
is already resident in HBM:
  * plan() + run() of the long paged prefill: one 32768-token prompt, no
    prefix, window_left 4095, 32 query / 8 KV heads, head_dim 128, page 16,
    bf16 (exact mask, per-tile KV-start skip);
  * plan() + run() of the large split-KV decode: 256 requests, kv_len
    U[1024, 32768], window_left 4095, 64 query / 8 KV heads, head_dim 128,
    page 16, bf16, 2048-key chunks merged from their (o, lse) partials.

Reported (one JSON line):
  value          window-effective prefill TFLOP/s: 4*D*H_q*sum_p n(p) FLOPs
                 (n(p) = keys visible to position p) over the prefill kernel's
                 average duration, measured with HIP events on the launch stream
  decode         KV-read GB/s of the decode run: sum_b H_kv*n_b*D*2B*2 bytes over
                 the decode run's duration (chunk kernel + merge kernel)
  roofline       prefill kernel against the bf16 dense MFMA peak
  roofline_decode  decode against the HBM peak
  cpu_baseline   the CPU oracle (single thread, fp64) on a bounded sample of
                 the prefill workload, in the same unit
  decode_no_window  the same decode batch with window_left -1, timed apart

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def prefill_flops(case) -> int:
    W = case.window_left
    total = 0
    for qo, kv in zip(case.qo_lens, case.kv_lens):
        prefix = kv - qo
        for p in range(prefix, kv):
            total += (min(p, W) + 1) if W >= 0 else (p + 1)
    return 4 * case.head_dim * case.num_qo_heads * total


def decode_bytes(case, W) -> int:
    n = sum((min(kv, W + 1) if W >= 0 else kv) for kv in case.kv_lens)
    return n * case.num_kv_heads * case.head_dim * 2 * 2


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_sliding_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = data.get(kernel)
    if not ent or ent.get("source_digest") != source_digest():
        return None
    return ent.get("hbm_bytes_per_launch")


def cpu_baseline(case, budget_s: float = 15.0):
    """Time the CPU oracle on a bounded sample of the prefill workload."""
    import numpy as np

    import oracle

    qcpu = case.q.cpu()
    kc, vc = case.k_cache.cpu(), case.v_cache.cpu()
    W = case.window_left
    rng = np.random.default_rng(0)
    rows, flops, elapsed = [], 0, 0.0
    # sample query tokens past the window (full W+1 keys each), a few at a time
    while elapsed < budget_s and len(rows) < 4096:
        batch = rng.integers(W, case.qo_lens[0], size=4).tolist()
        t0 = time.perf_counter()
        oracle.paged_attention(qcpu, kc, vc, case.qo_indptr, case.kv_indptr, case.kv_indices,
                               case.kv_last_page_len, num_qo_heads=case.num_qo_heads,
                               num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                               page_size=case.page_size, causal=True, window_left=W,
                               sm_scale=case.sm_scale, rows=batch)
        elapsed += time.perf_counter() - t0
        rows += batch
        flops += 4 * case.head_dim * case.num_qo_heads * (W + 1) * len(batch)
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{len(rows)} query tokens (all {case.num_qo_heads} heads, {W + 1} visible "
                   f"keys each) of the 32768-token prefill, fp64 C oracle, one thread, "
                   f"{elapsed:.1f} s"),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--only", choices=["prefill", "decode", "all"], default="all",
                    help="restrict the timed step (for profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only; multi-GPU sharding is a design "
              "note, not a code path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from paged_kv_sliding_amd import pkvs as P
    from paged_kv_sliding_amd.synth import build_case

    dev = "cuda"
    torch.cuda.set_device(0)
    print("bench: generating inputs", file=sys.stderr, flush=True)
    pre = build_case("long_prefill", device=dev)
    dec = build_case("split_decode", device=dev)
    W_dec = dec.window_left
    torch.cuda.synchronize()

    pre_att = P.BatchAttention(P.PKVS_PREFILL, num_qo_heads=pre.num_qo_heads,
                               num_kv_heads=pre.num_kv_heads, head_dim=pre.head_dim,
                               page_size=pre.page_size, dtype=pre.dtype,
                               window_left=pre.window_left, batch_capacity=1,
                               qo_capacity=pre.qo_lens[0], kv_capacity=pre.kv_lens[0])

    def dec_att(W):
        return P.BatchAttention(P.PKVS_DECODE, num_qo_heads=dec.num_qo_heads,
                                num_kv_heads=dec.num_kv_heads, head_dim=dec.head_dim,
                                page_size=dec.page_size, dtype=dec.dtype, window_left=W,
                                fixed_split_size=dec.fixed_split_size,
                                batch_capacity=dec.batch_size, kv_capacity=max(dec.kv_lens))

    dec_att_w = dec_att(W_dec)
    dec_att_full = dec_att(-1)
    o_pre = torch.empty_like(pre.q)
    l_pre = torch.empty(pre.q.shape[:2], dtype=torch.float32, device=dev)
    o_dec = torch.empty_like(dec.q)
    l_dec = torch.empty(dec.q.shape[:2], dtype=torch.float32, device=dev)
    pre_host = (pre.qo_indptr.cpu(), pre.kv_indptr.cpu(), pre.kv_last_page_len.cpu())
    dec_host = (dec.kv_indptr.cpu(), dec.kv_last_page_len.cpu())

    ev = {k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for k in ("pre", "dec")}
    times = {"pre": [], "dec": []}

    def step(record: bool):
        if args.only in ("prefill", "all"):
            pre_att.plan(qo_indptr=pre_host[0], kv_indptr=pre_host[1],
                         kv_last_page_len=pre_host[2])
            if record:
                ev["pre"][0].record()
            pre_att.run(pre.q, pre.k_cache, pre.v_cache, pre.kv_indices, sm_scale=pre.sm_scale,
                        window_left=pre.window_left, out=o_pre, lse=l_pre)
            if record:
                ev["pre"][1].record()
        if args.only in ("decode", "all"):
            dec_att_w.plan(kv_indptr=dec_host[0], kv_last_page_len=dec_host[1])
            if record:
                ev["dec"][0].record()
            dec_att_w.run(dec.q, dec.k_cache, dec.v_cache, dec.kv_indices, sm_scale=dec.sm_scale,
                          window_left=W_dec, out=o_dec, lse=l_dec)
            if record:
                ev["dec"][1].record()

    print("bench: warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    print(f"bench: timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
        torch.cuda.synchronize()
        for k in times:
            if (k == "pre" and args.only == "decode") or (k == "dec" and args.only == "prefill"):
                continue
            times[k].append(ev[k][0].elapsed_time(ev[k][1]))
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)

    res = {}
    flops = prefill_flops(pre)
    if times["pre"]:
        pre_ms = sum(times["pre"]) / len(times["pre"])
        tflops = flops / (pre_ms * 1e-3) / 1e12
        res["pre"] = (pre_ms, tflops)
    if times["dec"]:
        dec_ms = sum(times["dec"]) / len(times["dec"])
        nbytes = decode_bytes(dec, W_dec)
        res["dec"] = (dec_ms, nbytes / (dec_ms * 1e-3) / 1e9, nbytes)

    # the no-window decode of the same batch, timed apart (not part of the step)
    full = None
    if args.only == "all":
        dec_att_full.plan(kv_indptr=dec_host[0], kv_last_page_len=dec_host[1])
        for _ in range(2):
            dec_att_full.run(dec.q, dec.k_cache, dec.v_cache, dec.kv_indices,
                             sm_scale=dec.sm_scale, window_left=-1, out=o_dec, lse=l_dec)
        ts = []
        for _ in range(max(3, args.steps // 2)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            dec_att_full.run(dec.q, dec.k_cache, dec.v_cache, dec.kv_indices,
                             sm_scale=dec.sm_scale, window_left=-1, out=o_dec, lse=l_dec)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        ms = sum(ts) / len(ts)
        nb = decode_bytes(dec, -1)
        full = {"value": nb / (ms * 1e-3) / 1e9, "unit": "GB/s", "ms": round(ms, 4),
                "kv_bytes": nb, "frac_of_hbm_peak": nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS}

    line = {
        "metric": "SWA paged prefill TFLOP/s (window-effective) + decode KV GB/s, 1 GPU",
        "value": round(res["pre"][1], 2) if "pre" in res else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "swa_paged_step: prefill 1x32768 tokens W=4095 + decode 256 reqs "
                        "kv U[1024,32768] W=4095 split 2048",
            "prefill": {"batch": 1, "seq_len": 32768, "window_left": pre.window_left,
                        "num_qo_heads": 32, "num_kv_heads": 8, "head_dim": 128,
                        "page_size": 16, "window_effective_flops": flops},
            "decode": {"batch": 256, "kv_len": "U[1024,32768] seed 5", "window_left": W_dec,
                       "num_qo_heads": 64, "num_kv_heads": 8, "head_dim": 128, "page_size": 16,
                       "fixed_split_size": 2048},
        },
    }
    if "pre" in res:
        pre_ms, tflops = res["pre"]
        line["prefill_ms"] = round(pre_ms, 4)
        line["roofline"] = {"bound": "mfma", "achieved": round(tflops, 2),
                            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                            "traffic": load_traffic("prefill_bf16_kernel<128>"),
                            "kernel": "prefill_bf16_kernel<128>",
                            "work_per_launch": flops}
    if "dec" in res:
        dec_ms, gbps, nbytes = res["dec"]
        line["decode"] = {"value": round(gbps, 1), "unit": "GB/s", "ms": round(dec_ms, 4),
                          "kv_bytes": nbytes}
        line["roofline_decode"] = {"bound": "hbm", "achieved": round(gbps, 1),
                                   "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                   "frac": round(gbps / PEAK_HBM_GBPS, 4),
                                   "traffic": load_traffic("decode_bf16_kernel<128>"),
                                   "kernel": "decode_bf16_kernel<128> + decode_merge_kernel<128>",
                                   "work_per_launch": nbytes}
    if full is not None:
        line["decode_no_window"] = full
    if not args.no_cpu_baseline and args.only == "all":
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(pre, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
