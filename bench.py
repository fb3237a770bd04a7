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
  roofline       prefill kernel against the bf16 dense MFMA peak (the published
                 2.5 PFLOP/s; device_peak: CUs x peak clock x 4096 FLOP/clk/CU
                 from the device's properties, beside it)
  roofline_decode  decode against the HBM peak
  cpu_baseline   the CPU oracle (fp64, threads over query rows on the host's
                 cores) on a bounded sample of the prefill workload, in the same
                 unit; per_config times it on every workload in that
                 workload's unit (prefill GFLOP/s, decode KV GB/s)
  plan_host_us   host time of the plan() calls (median, microseconds)
  merge_state    the pairwise merge at the split decode's partial shape and
                 at 32768 tokens x 32 heads, HBM bytes 3*N*H*(D*2+4)
  decode_no_window  the same decode batch with window_left -1, timed apart
  cascade        the cascade prefill (new tokens' K/V contiguous, cached prefix
                 paged, merged), timed apart on two batches with cached
                 prefixes, beside the one paged prefill of the same batch
  pool           cache writes of a 32768-token prompt's K/V and the split
                 decode's page-table build, timed apart
  decode_fp8_kv  the split decode over an e4m3 copy of its cache, timed apart
  decode_sweep   the 64-request decode over its window sweep (W -1, 1023, 127,
                 31, 0), the last-level cache flushed before each timed run
Every GPU time is reported as the mean (which value and the rooflines use),
median and minimum over the timed launches; the last-level cache is flushed
(1 GiB written) before every timed decode launch, and a short spin kernel
keeps the GPU busy across each start event, so that the events time the
kernels and not the host's launch latency.

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
# the kernel the 32k-token prefill runs (the planner's choice for head_dim 128,
# bf16), as rocprofv3 names it, without the closing bracket
PREFILL_KERNEL = "prefill_big_kernel<false"
kXCDS = 8                   # XCDs of an MI355X (GRBM counters are summed over them)


# dense bf16 MFMA FLOPs per clock and CU on gfx950: 4 SIMDs, each finishing a
# 32x32x16 product (32768 FLOPs) every 32 clocks (the busy cycles rocprofv3
# counts per MFMA)
MFMA_BF16_FLOP_PER_CLK_CU = 4 * 1024


def device_peak() -> dict:
    """The bf16 dense MFMA peak from the device's own properties: compute units
    x peak engine clock (hipDeviceGetAttribute) x MFMA_BF16_FLOP_PER_CLK_CU."""
    import ctypes

    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    clk_khz = ctypes.c_int(0)
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        # hipDeviceAttributeClockRate: entry 5 of hipDeviceAttribute_t (ROCm 7
        # hip_runtime_api.h), the peak clock in kHz
        rc = hip.hipDeviceGetAttribute(ctypes.byref(clk_khz), 5, torch.cuda.current_device())
    except OSError:
        rc = -1
    if rc != 0 or clk_khz.value <= 0:
        return {"cus": cus, "max_clock_mhz": None, "tflops": None}
    tflops = cus * clk_khz.value * 1e3 * MFMA_BF16_FLOP_PER_CLK_CU / 1e12
    return {"cus": cus, "max_clock_mhz": round(clk_khz.value / 1e3), "tflops": round(tflops, 1)}


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


def time_stats(ts) -> dict:
    """Mean, median and minimum of a list of milliseconds."""
    srt = sorted(ts)
    return {"mean": sum(ts) / len(ts), "median": srt[len(srt) // 2], "min": srt[0]}


_SPIN_CYCLES = None


def keep_gpu_busy() -> None:
    """Enqueue a short spin kernel (about 0.1 ms) on torch's current stream.

    Called right before a start event is recorded: the host then enqueues the
    timed launch while the GPU is still spinning, so the event pair measures
    the timed kernels, not the host's launch latency (with an idle GPU the
    start event fires at once and the kernel only starts after the host has
    prepared and launched it)."""
    import torch

    global _SPIN_CYCLES
    if _SPIN_CYCLES is None:
        # calibrate: the spin counts GPU clock ticks, whose rate is not known here
        n = 100000
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(n)  # first call loads the kernel
        torch.cuda.synchronize()
        a.record()
        torch.cuda._sleep(n)
        b.record()
        torch.cuda.synchronize()
        per_ms = n / max(a.elapsed_time(b), 1e-3)
        _SPIN_CYCLES = max(1000, int(per_ms * 0.1))
    torch.cuda._sleep(_SPIN_CYCLES)


def timed_launches(fn, reps: int, flush=None) -> list:
    """HIP-event times (ms) of `reps` calls of fn on torch's current stream (the
    stream the binding launches on), each after an optional flush, with the
    GPU kept busy across the start event (keep_gpu_busy)."""
    import torch

    ts = []
    for _ in range(reps):
        if flush is not None:
            flush()
        keep_gpu_busy()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return ts


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_sliding_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(*kernels: str):
    """HBM bytes per launch (summed over `kernels`) from committed rocprofv3
    counter runs, if they were taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    total, digest = 0, source_digest()
    for kernel in kernels:
        ent = data.get(kernel)
        if not ent or ent.get("source_digest") != digest:
            return None
        total += ent["hbm_bytes_per_launch"]
    return total


def prefill_algorithmic_bytes(case) -> int:
    """Compulsory HBM bytes of one prefill launch: Q read once, the K and V rows
    the queries can see read once, O written once (same dtype), LSE in fp32."""
    W = case.window_left
    esz = case.q.element_size()
    kv_rows = 0
    for qo, kv in zip(case.qo_lens, case.kv_lens):
        first = max(0, kv - qo - W) if W >= 0 else 0
        kv_rows += kv - first
    tokens = sum(case.qo_lens)
    return (2 * tokens * case.num_qo_heads * case.head_dim * esz
            + 2 * kv_rows * case.num_kv_heads * case.head_dim * esz
            + tokens * case.num_qo_heads * 4)


COPY_BYTES = 1 << 30        # calibration copy: 1 GiB read + 1 GiB written


CASCADE_WORKLOADS = {
    # 8 requests, prefix U[0,1024], U[1,512] new tokens, W 511, head_dim 256
    "prefix_prefill": None,
    # the last 8192 tokens of a 32768-token prompt over its cached 24576
    "chunk_8192_after_24576": dict(qo=[8192], kv=[32768], H_q=32, H_kv=8, D=128, P=16,
                                   W=4095, seed=6),
    # a 1024-token chunk of a prompt over its cached 8192: 128 query tiles of
    # 64 tokens for 256 workgroups, so the plan cuts their key ranges
    "chunk_1024_after_8192": dict(qo=[1024], kv=[9216], H_q=32, H_kv=8, D=128, P=16, W=4095,
                                  seed=7),
}


def bench_cascade(reps: int) -> dict:
    """Cascade prefill beside the one paged prefill of the same batch, both
    timed with HIP events around run() on the launch stream, in alternation."""
    import torch

    from paged_kv_sliding_amd import pkvs as P
    from paged_kv_sliding_amd.synth import build_case, cascade_inputs, case_from_lengths

    out = {}
    for name, w in CASCADE_WORKLOADS.items():
        if w is None:
            c = build_case(name, device="cuda")
        else:
            c = case_from_lengths(name, w["qo"], w["kv"], num_qo_heads=w["H_q"],
                                  num_kv_heads=w["H_kv"], head_dim=w["D"], page_size=w["P"],
                                  dtype=torch.bfloat16, window_left=w["W"], seed=w["seed"],
                                  device="cuda")
        W = c.window_left
        ci = cascade_inputs(c, trim_to=W)
        kw = dict(num_qo_heads=c.num_qo_heads, num_kv_heads=c.num_kv_heads,
                  head_dim=c.head_dim, page_size=c.page_size, dtype=c.dtype, window_left=W,
                  batch_capacity=c.batch_size, qo_capacity=sum(c.qo_lens))
        cas = P.CascadeAttention(kv_capacity=max(max(ci.table_lens), 1), **kw)
        cas.plan(qo_indptr=c.qo_indptr.cpu(), kv_indptr=ci.kv_indptr,
                 kv_last_page_len=ci.kv_last_page_len)
        one = P.BatchAttention(P.PKVS_PREFILL, kv_capacity=max(c.kv_lens), **kw)
        one.plan(qo_indptr=c.qo_indptr.cpu(), kv_indptr=c.kv_indptr.cpu(),
                 kv_last_page_len=c.kv_last_page_len.cpu())
        o = torch.empty_like(c.q)
        lse = torch.empty(c.q.shape[:2], dtype=torch.float32, device="cuda")

        def run_cascade():
            cas.run(c.q, ci.k_extend, ci.v_extend, ci.k_cache, ci.v_cache, ci.kv_indices,
                    sm_scale=c.sm_scale, window_left=W, out=o, lse=lse)

        def run_one():
            one.run(c.q, c.k_cache, c.v_cache, c.kv_indices, sm_scale=c.sm_scale,
                    window_left=W, out=o, lse=lse)

        # warmed and timed in alternation, so that neither side gets the
        # clock's ramp or a colder cache than the other
        for _ in range(10):
            run_cascade()
            run_one()
        ts = {"cascade": [], "paged": []}
        for _ in range(reps):
            ts["cascade"] += timed_launches(run_cascade, 1)
            ts["paged"] += timed_launches(run_one, 1)
        res = {tag: time_stats(t) for tag, t in ts.items()}
        flops = prefill_flops(c)
        out[name] = {"ms": round(res["cascade"]["mean"], 4),
                     "ms_median": round(res["cascade"]["median"], 4),
                     "ms_min": round(res["cascade"]["min"], 4),
                     "tflops": round(flops / (res["cascade"]["mean"] * 1e-3) / 1e12, 2),
                     "paged_prefill_ms": round(res["paged"]["mean"], 4),
                     "paged_prefill_ms_median": round(res["paged"]["median"], 4),
                     "window_effective_flops": flops,
                     "prefill_variant": cas.info().prefill_variant,
                     # (token, kv head) rows merged after a key split: cascade, paged
                     "key_split_merges": [cas.info().num_merges, one.info().num_merges],
                     "batch": c.batch_size, "new_tokens": sum(c.qo_lens),
                     "cached_keys_in_tables": sum(ci.table_lens)}
        del ci, c
        torch.cuda.empty_cache()
    return out


def bench_decode_fp8(dec, W: int, reps: int, flush) -> dict:
    """The split decode batch over an e4m3 copy of its cache (K / k_scale,
    V / v_scale, converted in chunks on the device), same plan otherwise; KV
    bytes counted at one byte per element."""
    import torch

    from paged_kv_sliding_amd import pkvs as P

    ks, vs = 0.0625, 0.0625
    k8 = torch.empty(dec.k_cache.shape, dtype=torch.float8_e4m3fn, device="cuda")
    v8 = torch.empty_like(k8)
    step = 16384
    for i in range(0, k8.shape[0], step):
        k8[i:i + step] = (dec.k_cache[i:i + step].float() / ks).to(torch.float8_e4m3fn)
        v8[i:i + step] = (dec.v_cache[i:i + step].float() / vs).to(torch.float8_e4m3fn)
    att = P.BatchAttention(P.PKVS_DECODE, num_qo_heads=dec.num_qo_heads,
                           num_kv_heads=dec.num_kv_heads, head_dim=dec.head_dim,
                           page_size=dec.page_size, dtype=dec.dtype, window_left=W,
                           fixed_split_size=dec.fixed_split_size, batch_capacity=dec.batch_size,
                           kv_capacity=max(dec.kv_lens), kv_dtype=torch.float8_e4m3fn)
    att.plan(kv_indptr=dec.kv_indptr.cpu(), kv_last_page_len=dec.kv_last_page_len.cpu())
    o = torch.empty_like(dec.q)
    lse = torch.empty(dec.q.shape[:2], dtype=torch.float32, device="cuda")

    def run():
        att.run(dec.q, k8, v8, dec.kv_indices, sm_scale=dec.sm_scale, window_left=W, out=o,
                lse=lse, k_scale=ks, v_scale=vs)

    for _ in range(3):
        run()
    st = time_stats(timed_launches(run, reps, flush))
    ms = st["mean"]
    nb = decode_bytes(dec, W) // 2
    del k8, v8
    torch.cuda.empty_cache()
    return {"format": "e4m3", "ms": round(ms, 4), "ms_median": round(st["median"], 4),
            "ms_min": round(st["min"], 4), "kv_bytes": nb,
            "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}


def bench_decode_sweep(reps: int) -> dict:
    """The 64-request decode (kv U[1,4096], 32/8 heads, head_dim 128) over its
    window sweep.  Its K/V (0.26-537 MB) fit the 256 MB last-level cache, so
    before each timed run 1 GiB is written to flush it; each run is timed
    apart with HIP events around run()."""
    import torch

    from paged_kv_sliding_amd import pkvs as P
    from paged_kv_sliding_amd.synth import build_case

    c = build_case("decode_sweep", device="cuda")
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(c.q)
    lse = torch.empty(c.q.shape[:2], dtype=torch.float32, device="cuda")
    out = {}
    for W in (-1, 1023, 127, 31, 0):
        att = P.BatchAttention(P.PKVS_DECODE, num_qo_heads=c.num_qo_heads,
                               num_kv_heads=c.num_kv_heads, head_dim=c.head_dim,
                               page_size=c.page_size, dtype=c.dtype, window_left=W,
                               batch_capacity=c.batch_size, kv_capacity=max(c.kv_lens))
        att.plan(kv_indptr=c.kv_indptr.cpu(), kv_last_page_len=c.kv_last_page_len.cpu())

        def run():
            att.run(c.q, c.k_cache, c.v_cache, c.kv_indices, sm_scale=c.sm_scale,
                    window_left=W, out=o, lse=lse)

        for _ in range(3):
            run()
        st = time_stats(timed_launches(run, reps, lambda: flush.fill_(1)))
        ms = st["median"]
        nb = decode_bytes(c, W)
        out[f"W{W}"] = {"ms_median": round(ms, 4), "ms_min": round(st["min"], 4),
                        "ms_mean": round(st["mean"], 4), "kv_bytes": nb,
                        "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
                        "frac_of_hbm_peak": round(nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                        "split_size": att.info().split_size, "items": att.info().num_items}
        att.close()
    del flush
    torch.cuda.empty_cache()
    return out


def bench_pool(reps: int) -> dict:
    """The steps on either side of the attention: writing a 32768-token
    prompt's keys and values into its pages (slot = page * 16 + position, the
    long prefill's own page table) and building the split decode's page table
    (256 requests, up to 2048 pages each) from a request-to-page map.  HIP
    events around each call on the launch stream."""
    import torch

    from paged_kv_sliding_amd import pkvs as P

    def timed(fn):
        for _ in range(3):
            fn()
        return time_stats(timed_launches(fn, reps))["mean"]

    out = {}
    g = torch.Generator(device="cuda").manual_seed(41)
    n, H, D, Psz = 32768, 8, 128, 16
    pages = torch.randperm(n // Psz, device="cuda")
    pos = torch.arange(n, device="cuda")
    loc = (pages[pos // Psz] * Psz + pos % Psz).to(torch.int64)
    k_new = torch.randn(n, H, D, generator=g, device="cuda").to(torch.bfloat16)
    v_new = torch.randn(n, H, D, generator=g, device="cuda").to(torch.bfloat16)
    kc = torch.empty(n // Psz, Psz, H, D, dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    ms = timed(lambda: P.pkvs_append_kv(k_new, v_new, loc, kc, vc))
    nbytes = 2 * 2 * n * H * D * 2  # K and V rows, read once and written once
    out["kv_append"] = {"rows": n, "row_bytes": H * D * 2, "ms": round(ms, 4),
                        "bytes": nbytes, "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                        "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
    k8 = torch.empty(kc.shape, dtype=torch.float8_e4m3fn, device="cuda")
    v8 = torch.empty_like(k8)
    ms = timed(lambda: P.pkvs_append_kv(k_new, v_new, loc, k8, v8, k_scale=0.0625,
                                        v_scale=0.0625))
    nbytes = 2 * n * H * D * (2 + 1)  # bf16 rows read, e4m3 rows written
    out["kv_append_e4m3"] = {"rows": n, "ms": round(ms, 4), "bytes": nbytes,
                             "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    del k_new, v_new, kc, vc, k8, v8
    gen = torch.Generator().manual_seed(5)
    kv = torch.randint(1024, 32769, (256,), generator=gen)
    npg = ((kv + 15) // 16).to(torch.int32)
    page_map = torch.randint(0, 1 << 20, (256, 2048), dtype=torch.int32, device="cuda")
    slot = torch.randperm(256, device="cuda").to(torch.int32)
    length = npg.to("cuda")
    cap = int(npg.sum())
    kp = torch.empty(257, dtype=torch.int32, device="cuda")
    ki = torch.empty(cap, dtype=torch.int32, device="cuda")
    ms = timed(lambda: P.pkvs_build_kv_indices(page_map, slot, length, kv_indptr=kp,
                                               kv_indices=ki, capacity=cap))
    out["page_table_build"] = {"requests": 256, "entries": cap, "ms": round(ms, 4),
                               "bytes": cap * 8 + 256 * 12}
    return out


MERGE_SHAPES = {
    # the split decode's partials: one (o, lse) pair per request and query head
    "split_decode_partials": (256, 64, 128),
    # a long prefill's two halves: 32768 tokens x 32 heads
    "tokens_32768_heads_32": (32768, 32, 128),
}


def bench_merge_state(reps: int, flush) -> dict:
    """pkvs_merge_state on bf16 v and fp32 s: bytes = 3*N*H*(D*2 + 4) (two
    partials read, one written), HIP events around each call, the last-level
    cache flushed before each."""
    import torch

    from paged_kv_sliding_amd import pkvs as P

    out = {}
    g = torch.Generator(device="cuda").manual_seed(17)
    for name, (n, h, d) in MERGE_SHAPES.items():
        va = torch.randn(n, h, d, generator=g, device="cuda").to(torch.bfloat16)
        vb = torch.randn(n, h, d, generator=g, device="cuda").to(torch.bfloat16)
        sa = torch.randn(n, h, generator=g, device="cuda") * 4
        sb = torch.randn(n, h, generator=g, device="cuda") * 4
        vo, so = torch.empty_like(va), torch.empty_like(sa)

        def run():
            P.pkvs_merge_state(va, sa, vb, sb, v_out=vo, s_out=so)

        for _ in range(3):
            run()
        st = time_stats(timed_launches(run, reps, flush))
        nb = 3 * n * h * (d * 2 + 4)
        gbps = nb / (st["mean"] * 1e-3) / 1e9
        out[name] = {"tokens": n, "heads": h, "head_dim": d, "v_dtype": "bf16",
                     "ms": round(st["mean"], 4), "ms_median": round(st["median"], 4),
                     "ms_min": round(st["min"], 4), "bytes": nb, "GB/s": round(gbps, 1),
                     "frac_of_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4)}
        del va, vb, sa, sb, vo, so
    torch.cuda.empty_cache()
    return out


def profile_kernel(which: str, reps: int) -> None:
    """Launch one kernel `reps` times and nothing else timed, for rocprofv3
    counter passes; prints the source digest the counters belong to."""
    import torch

    from paged_kv_sliding_amd import pkvs as P
    from paged_kv_sliding_amd.synth import build_case

    torch.cuda.set_device(0)
    print(f"source_digest={source_digest()}", flush=True)
    if which == "copy":
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(7)
        dst = torch.empty_like(src)
        for _ in range(reps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copy bytes={COPY_BYTES} reps={reps}", flush=True)
        return
    name = "long_prefill" if which == "prefill" else "split_decode"
    c = build_case(name, device="cuda")
    att = P.BatchAttention(P.PKVS_PREFILL if which == "prefill" else P.PKVS_DECODE,
                           num_qo_heads=c.num_qo_heads, num_kv_heads=c.num_kv_heads,
                           head_dim=c.head_dim, page_size=c.page_size, dtype=c.dtype,
                           window_left=c.window_left, fixed_split_size=c.fixed_split_size,
                           batch_capacity=c.batch_size, qo_capacity=sum(c.qo_lens),
                           kv_capacity=max(c.kv_lens))
    if which == "prefill":
        att.plan(qo_indptr=c.qo_indptr.cpu(), kv_indptr=c.kv_indptr.cpu(),
                 kv_last_page_len=c.kv_last_page_len.cpu())
    else:
        att.plan(kv_indptr=c.kv_indptr.cpu(), kv_last_page_len=c.kv_last_page_len.cpu())
    o = torch.empty_like(c.q)
    lse = torch.empty(c.q.shape[:2], dtype=torch.float32, device="cuda")
    for _ in range(reps):
        att.run(c.q, c.k_cache, c.v_cache, c.kv_indices, sm_scale=c.sm_scale,
                window_left=c.window_left, out=o, lse=lse)
    torch.cuda.synchronize()
    alg = prefill_algorithmic_bytes(c) if which == "prefill" else decode_bytes(c, c.window_left)
    print(f"{which} workload={name} reps={reps} algorithmic_bytes={alg}", flush=True)


def _counter_means(csv_path: str, counter: str) -> dict:
    """Mean per-dispatch value of `counter` for each kernel in a rocprofv3
    counter_collection.csv."""
    import csv

    acc = {}
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            acc.setdefault(name, []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}


def ingest_counters(d: str) -> None:
    """Turn the FETCH_SIZE / WRITE_SIZE passes under `d` into HBM bytes per
    launch, calibrated by the plain 1 GiB copy, and write profiles/traffic.json."""
    import glob

    digest = source_digest()
    for out in glob.glob(os.path.join(d, "*.out")):
        for ln in open(out):
            if ln.startswith("source_digest=") and ln.strip().split("=")[1] != digest:
                sys.exit(f"ingest: {out} was taken on other kernel sources; run the passes again")

    def pass_means(kind, ctr):
        path = os.path.join(d, f"{ctr.lower()}_{kind}", "p_counter_collection.csv")
        return _counter_means(path, ctr)

    def pick(means, key):
        names = [n for n in means[0] if key in n]
        if len(names) != 1:
            sys.exit(f"ingest: expected one kernel matching {key!r}, found {names}")
        return names[0]

    # calibration: KiB the counters report for a copy of COPY_BYTES in and out
    cal = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        m = pass_means("copy", ctr)
        n = pick(m, "copyBuffer")
        cal[ctr] = COPY_BYTES / (m[0][n] * 1024.0)
    res = {"calibration": {"copy_bytes": COPY_BYTES,
                           "fetch_factor": round(cal["FETCH_SIZE"], 4),
                           "write_factor": round(cal["WRITE_SIZE"], 4)}}
    for kind, kernels in (("prefill", [PREFILL_KERNEL]),
                          ("decode", ["decode_kernel<128", "decode_merge_kernel<128"])):
        fm, wm = pass_means(kind, "FETCH_SIZE"), pass_means(kind, "WRITE_SIZE")
        for key in kernels:
            nf, nw = pick(fm, key), pick(wm, key)
            fetch = fm[0][nf] * 1024.0 * cal["FETCH_SIZE"]
            write = wm[0][nw] * 1024.0 * cal["WRITE_SIZE"]
            res[key + ">"] = {"source_digest": digest, "dispatches": fm[1][nf],
                              "fetch_bytes_per_launch": int(fetch),
                              "write_bytes_per_launch": int(write),
                              "hbm_bytes_per_launch": int(fetch + write)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res, indent=1))


# rocprofv3 --pmc passes for the prefill kernel's execution counters (each
# within one pass's limits: at most 8 SQ and 2 GRBM counters)
PREFILL_COUNTER_PASSES = {
    "issue": ["SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
              "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_ANY", "SQ_LDS_CMD_FIFO_FULL", "GRBM_GUI_ACTIVE",
              "GRBM_COUNT"],
    "insts": ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU",
              "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_ACTIVE_INST_VALU",
              "SQ_ACTIVE_INST_LDS", "GRBM_GUI_ACTIVE"],
    "lds": ["SQ_INSTS_VALU_TRANS_F32", "SQ_LDS_DATA_FIFO_FULL", "SQ_LDS_BANK_CONFLICT",
            "SQ_INST_LEVEL_LDS", "SQ_BUSY_CU_CYCLES", "SQ_ACTIVE_INST_SCA", "SQ_INSTS_SMEM",
            "SQ_INSTS_VMEM", "GRBM_GUI_ACTIVE"],
}


def summarize_prefill_counters(d: str, out_md: str) -> None:
    """Turn the PREFILL_COUNTER_PASSES runs under `d` (one rocprofv3 --pmc run
    of `bench.py --profile-kernel prefill` per pass, in d/<pass>/p_*) into a
    markdown summary of the prefill kernel's per-launch counters."""
    import glob

    digest = source_digest()
    for out in glob.glob(os.path.join(d, "*.out")):
        for ln in open(out):
            if ln.startswith("source_digest=") and ln.strip().split("=")[1] != digest:
                sys.exit(f"summarize: {out} was taken on other kernel sources")
    vals, n_disp = {}, None
    for pas, ctrs in PREFILL_COUNTER_PASSES.items():
        path = os.path.join(d, pas, "p_counter_collection.csv")
        for ctr in ctrs:
            means, counts = _counter_means(path, ctr)
            names = [k for k in means if PREFILL_KERNEL in k]
            if len(names) != 1:
                sys.exit(f"summarize: {ctr}: expected one prefill kernel in {path}, got {names}")
            vals.setdefault(ctr, means[names[0]])
            n_disp = counts[names[0]]
    props = {}
    try:
        import torch

        pr = torch.cuda.get_device_properties(0)
        props = {"cus": pr.multi_processor_count}
    except Exception:
        pass
    cus = props.get("cus", 256)
    simds = 4 * cus
    xcd_cycles = vals["GRBM_GUI_ACTIVE"] / kXCDS
    mfma = vals["SQ_INSTS_MFMA"]
    rows = [
        ("launches measured (mean per launch below)", f"{n_disp}"),
        ("GRBM_GUI_ACTIVE / 8 (GPU cycles of one XCD)", f"{xcd_cycles:,.0f}"),
        ("MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x XCD cycles)",
         f"{vals['SQ_VALU_MFMA_BUSY_CYCLES'] / (simds * xcd_cycles):.3f}"),
        ("VALU and MFMA co-issued: SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES",
         f"{vals['SQ_VALU_MFMA_COEXEC_CYCLES'] / vals['SQ_VALU_MFMA_BUSY_CYCLES']:.3f}"),
        ("SQ_INSTS_MFMA", f"{mfma:,.0f}"),
        ("SQ_INSTS_VALU (MFMA included) / SQ_INSTS_MFMA",
         f"{vals['SQ_INSTS_VALU'] / mfma:.2f}"),
        ("(SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA",
         f"{(vals['SQ_INSTS_VALU'] - mfma) / mfma:.2f}"),
        ("SQ_INSTS_VALU_TRANS_F32 / SQ_INSTS_MFMA",
         f"{vals['SQ_INSTS_VALU_TRANS_F32'] / mfma:.2f}"),
        ("SQ_INSTS_LDS / SQ_INSTS_MFMA", f"{vals['SQ_INSTS_LDS'] / mfma:.2f}"),
        ("SQ_INSTS_SALU / SQ_INSTS_MFMA", f"{vals['SQ_INSTS_SALU'] / mfma:.2f}"),
        ("SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES",
         f"{vals['SQ_WAIT_INST_LDS'] / vals['SQ_WAVE_CYCLES']:.3f}"),
        ("SQ_WAIT_ANY / SQ_WAVE_CYCLES", f"{vals['SQ_WAIT_ANY'] / vals['SQ_WAVE_CYCLES']:.3f}"),
        ("SQ_ACTIVE_INST_LDS / SQ_WAVE_CYCLES",
         f"{vals['SQ_ACTIVE_INST_LDS'] / vals['SQ_WAVE_CYCLES']:.3f}"),
        ("SQ_LDS_CMD_FIFO_FULL", f"{vals['SQ_LDS_CMD_FIFO_FULL']:,.0f}"),
        ("SQ_LDS_DATA_FIFO_FULL", f"{vals['SQ_LDS_DATA_FIFO_FULL']:,.0f}"),
        ("SQ_LDS_BANK_CONFLICT", f"{vals['SQ_LDS_BANK_CONFLICT']:,.0f}"),
    ]
    lines = [f"# Execution counters: `{PREFILL_KERNEL}>` on the 32768-token prefill", "",
             "Workload: one request, 32768 query tokens, no prefix, window_left 4095, "
             "32 query / 8 KV heads, head_dim 128, page_size 16, bf16.",
             f"Kernel sources at digest `{digest}`.  Device: {cus} CUs, {simds} SIMDs.", "",
             "Commands (from the repository root, on a machine with the MI355X; one pass per run):", "", "```"]
    for pas, ctrs in PREFILL_COUNTER_PASSES.items():
        lines.append(f"rocprofv3 --pmc {' '.join(ctrs)} -d <dir>/{pas} -o p --output-format csv "
                     f"-- python3 bench.py --profile-kernel prefill --reps 5")
    lines += [f"python3 bench.py --summarize-counters <dir>", "```", "",
              "| quantity | per launch |", "|---|---|"]
    lines += [f"| {k} | {v} |" for k, v in rows]
    lines += ["", "Raw means per launch:", "", "| counter | value |", "|---|---|"]
    lines += [f"| {k} | {v:,.0f} |" for k, v in sorted(vals.items())]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def window_sample(case, requests, W: int):
    """The listed decode requests of `case` as a host case holding only the
    pages their window reaches: the dropped leading pages hold no visible key,
    and the query keeps its place relative to the kept keys."""
    import dataclasses

    import torch

    P = case.page_size
    kvp, idx = case.kv_indptr.cpu(), case.kv_indices.cpu()
    pages, npg, lens, last = [], [], [], []
    for b in requests:
        n = case.kv_lens[b]
        drop = max(0, n - 1 - W) // P if W >= 0 else 0
        pg = idx[int(kvp[b]) + drop:int(kvp[b + 1])]
        pages.append(pg)
        npg.append(len(pg))
        lens.append(n - drop * P)
        last.append(int(case.kv_last_page_len[b]))
    pages = torch.cat(pages).long().to(case.k_cache.device)
    kvp2 = torch.zeros(len(requests) + 1, dtype=torch.int32)
    kvp2[1:] = torch.tensor(npg).cumsum(0)
    return dataclasses.replace(
        case, qo_lens=[1] * len(requests), kv_lens=lens,
        q=case.q[torch.tensor(list(requests), device=case.q.device)].cpu(),
        k_cache=case.k_cache.index_select(0, pages).cpu(),
        v_cache=case.v_cache.index_select(0, pages).cpu(),
        qo_indptr=torch.arange(len(requests) + 1, dtype=torch.int32), kv_indptr=kvp2,
        kv_indices=torch.arange(int(kvp2[-1]), dtype=torch.int32),
        kv_last_page_len=torch.tensor(last, dtype=torch.int32), window_left=W)


def cpu_baseline(pre, dec, budget_s: float = 10.0) -> dict:
    """The CPU oracle (fp64, query rows spread over the host cores it is given)
    timed on every workload, each in that workload's unit: the whole 8-request
    prefix prefill, the whole 64-request decode at W -1 and 1023, a sample of
    the 32768-token prefill's query tokens (about budget_s seconds) and a sample
    of the 256-request decode's requests.  The top-level value is the long
    prefill sample, in the unit of the bench's value."""
    import numpy as np

    import oracle
    from paged_kv_sliding_amd.synth import build_case

    threads = oracle.default_threads()
    per = {}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    c2 = build_case("prefix_prefill", device="cpu")
    dt = timed(lambda: oracle.case_attention(c2, threads=threads))
    per["prefix_prefill"] = {"value": round(prefill_flops(c2) / dt / 1e9, 3), "unit": "GFLOP/s",
                             "seconds": round(dt, 3), "sample": "the whole 8-request batch"}
    c3 = build_case("decode_sweep", device="cpu")
    for W in (-1, 1023):
        dt = timed(lambda: oracle.case_attention(c3, window_left=W, threads=threads))
        per[f"decode_sweep_W{W}"] = {"value": round(decode_bytes(c3, W) / dt / 1e9, 3),
                                     "unit": "GB/s (K/V read)", "seconds": round(dt, 3),
                                     "sample": "all 64 requests"}
    del c2, c3

    # long prefill: query tokens past the window (W+1 keys each), a batch of
    # 4 rows per thread at a time, until the budget is spent
    qcpu, kc, vc = pre.q.cpu(), pre.k_cache.cpu(), pre.v_cache.cpu()
    W = pre.window_left
    rng = np.random.default_rng(0)
    rows, flops, elapsed = 0, 0, 0.0
    while elapsed < budget_s and rows < 32768:
        batch = rng.integers(W, pre.qo_lens[0], size=4 * threads).tolist()
        elapsed += timed(lambda: oracle.paged_attention(
            qcpu, kc, vc, pre.qo_indptr, pre.kv_indptr, pre.kv_indices, pre.kv_last_page_len,
            num_qo_heads=pre.num_qo_heads, num_kv_heads=pre.num_kv_heads,
            head_dim=pre.head_dim, page_size=pre.page_size, causal=True, window_left=W,
            sm_scale=pre.sm_scale, rows=batch, threads=threads))
        rows += len(batch)
        flops += 4 * pre.head_dim * pre.num_qo_heads * (W + 1) * len(batch)
    del qcpu, kc, vc
    long_rate = flops / elapsed
    per["long_prefill"] = {"value": round(long_rate / 1e9, 3), "unit": "GFLOP/s",
                           "seconds": round(elapsed, 3),
                           "sample": f"{rows} query tokens (all {pre.num_qo_heads} heads, {W + 1} "
                                     f"visible keys each) of the {pre.qo_lens[0]} tokens"}

    # split decode, W = 4095: 4 requests per thread, only the pages each window reaches
    Wd = dec.window_left
    picks = sorted(np.random.default_rng(5).choice(dec.batch_size, size=min(dec.batch_size,
                                                                              4 * threads),
                                                   replace=False).tolist())
    sub = window_sample(dec, picks, Wd)
    dt = timed(lambda: oracle.case_attention(sub, threads=threads))
    per[f"split_decode_W{Wd}"] = {"value": round(decode_bytes(sub, Wd) / dt / 1e9, 3),
                                  "unit": "GB/s (K/V read)", "seconds": round(dt, 3),
                                  "sample": f"{len(picks)} of the {dec.batch_size} requests"}
    return {
        "value": long_rate / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": per["long_prefill"]["sample"] + f", fp64 C oracle, {threads} threads, "
                                                  f"{elapsed:.1f} s",
        "per_config": per,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--only", choices=["prefill", "decode", "cascade", "pool", "sweep", "merge",
                                       "cpu", "all"],
                    default="all",
                    help="restrict the timed step (for profiling runs)")
    ap.add_argument("--profile-kernel", choices=["prefill", "decode", "copy"],
                    help="launch only this kernel --reps times (rocprofv3 counter passes)")
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--prefill-variant", type=int, default=0,
                    help="prefill kernel variant of the long prefill (0: the planner's choice)")
    ap.add_argument("--ingest-counters", metavar="DIR",
                    help="write profiles/traffic.json from FETCH_SIZE/WRITE_SIZE passes in DIR")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="write profiles/prefill_counters.md from the PREFILL_COUNTER_PASSES "
                         "runs in DIR")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(args.ingest_counters)
        return
    if args.summarize_counters:
        summarize_prefill_counters(args.summarize_counters,
                                   os.path.join(ROOT, "profiles", "prefill_counters.md"))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only; multi-GPU sharding is a design "
              "note, not a code path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.profile_kernel:
        profile_kernel(args.profile_kernel, args.reps)
        return

    if args.only == "cascade":
        print(json.dumps({"cascade": bench_cascade(args.steps)}), flush=True)
        return
    if args.only == "pool":
        print(json.dumps({"pool": bench_pool(args.steps)}), flush=True)
        return
    if args.only == "sweep":
        print(json.dumps({"decode_sweep": bench_decode_sweep(args.steps)}), flush=True)
        return
    if args.only == "merge":
        import torch

        buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        print(json.dumps({"merge_state": bench_merge_state(args.steps, lambda: buf.fill_(1))}),
              flush=True)
        return

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
                               qo_capacity=pre.qo_lens[0], kv_capacity=pre.kv_lens[0],
                               prefill_variant=args.prefill_variant)

    def dec_att(W):
        return P.BatchAttention(P.PKVS_DECODE, num_qo_heads=dec.num_qo_heads,
                                num_kv_heads=dec.num_kv_heads, head_dim=dec.head_dim,
                                page_size=dec.page_size, dtype=dec.dtype, window_left=W,
                                fixed_split_size=dec.fixed_split_size,
                                batch_capacity=dec.batch_size, kv_capacity=max(dec.kv_lens))

    if args.only == "cpu":
        print(json.dumps({"cpu_baseline": cpu_baseline(pre, dec, args.cpu_budget)}), flush=True)
        return
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
    plan_us = {"pre": [], "dec": []}
    # written before every timed decode launch: the 64-request decode's K/V
    # (up to 0.6 GB) and part of the 4 GB split decode would otherwise be
    # served from the 256 MB last-level cache
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def flush():
        flush_buf.fill_(1)

    def step(record: bool):
        if args.only in ("prefill", "all"):
            t0 = time.perf_counter()
            pre_att.plan(qo_indptr=pre_host[0], kv_indptr=pre_host[1],
                         kv_last_page_len=pre_host[2])
            if record:
                plan_us["pre"].append((time.perf_counter() - t0) * 1e6)
                keep_gpu_busy()
                ev["pre"][0].record()
            pre_att.run(pre.q, pre.k_cache, pre.v_cache, pre.kv_indices, sm_scale=pre.sm_scale,
                        window_left=pre.window_left, out=o_pre, lse=l_pre)
            if record:
                ev["pre"][1].record()
        if args.only in ("decode", "all"):
            flush()
            t0 = time.perf_counter()
            dec_att_w.plan(kv_indptr=dec_host[0], kv_last_page_len=dec_host[1])
            if record:
                plan_us["dec"].append((time.perf_counter() - t0) * 1e6)
                keep_gpu_busy()
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
        st = time_stats(times["pre"])
        res["pre"] = (st, flops / (st["mean"] * 1e-3) / 1e12)
    if times["dec"]:
        st = time_stats(times["dec"])
        nbytes = decode_bytes(dec, W_dec)
        res["dec"] = (st, nbytes / (st["mean"] * 1e-3) / 1e9, nbytes)

    # the no-window decode of the same batch, timed apart (not part of the step)
    full = None
    fp8 = None
    if args.only == "all":
        print("bench: decode over an 8-bit cache", file=sys.stderr, flush=True)
        fp8 = bench_decode_fp8(dec, W_dec, max(5, args.steps // 2), flush)
        dec_att_full.plan(kv_indptr=dec_host[0], kv_last_page_len=dec_host[1])

        def run_full():
            dec_att_full.run(dec.q, dec.k_cache, dec.v_cache, dec.kv_indices,
                             sm_scale=dec.sm_scale, window_left=-1, out=o_dec, lse=l_dec)

        for _ in range(2):
            run_full()
        st = time_stats(timed_launches(run_full, max(3, args.steps // 2), flush))
        ms = st["mean"]
        nb = decode_bytes(dec, -1)
        full = {"value": nb / (ms * 1e-3) / 1e9, "unit": "GB/s", "ms": round(ms, 4),
                "ms_median": round(st["median"], 4), "ms_min": round(st["min"], 4),
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
        st, tflops = res["pre"]
        pre_ms = st["mean"]
        line["prefill_ms"] = round(pre_ms, 4)
        line["prefill_ms_median"] = round(st["median"], 4)
        line["prefill_ms_min"] = round(st["min"], 4)
        line["prefill_variant"] = pre_att.info().prefill_variant
        line["roofline"] = {"bound": "mfma", "achieved": round(tflops, 2),
                            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                            "traffic": load_traffic(PREFILL_KERNEL + ">"),
                            "algorithmic_bytes": prefill_algorithmic_bytes(pre),
                            "kernel": PREFILL_KERNEL + ">",
                            "work_per_launch": flops,
                            "device_peak": device_peak()}
    if "dec" in res:
        st, gbps, nbytes = res["dec"]
        line["decode"] = {"value": round(gbps, 1), "unit": "GB/s", "ms": round(st["mean"], 4),
                          "ms_median": round(st["median"], 4), "ms_min": round(st["min"], 4),
                          "kv_bytes": nbytes, "llc_flushed": True}
        line["roofline_decode"] = {"bound": "hbm", "achieved": round(gbps, 1),
                                   "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                   "frac": round(gbps / PEAK_HBM_GBPS, 4),
                                   "traffic": load_traffic("decode_kernel<128>",
                                                           "decode_merge_kernel<128>"),
                                   "kernel": "decode_kernel<128> + decode_merge_kernel<128>",
                                   "work_per_launch": nbytes}
    line["plan_host_us"] = {k2: round(time_stats(v)["median"], 1)
                            for k2, v in (("prefill", plan_us["pre"]), ("decode", plan_us["dec"]))
                            if v}
    if full is not None:
        line["decode_no_window"] = full
    if fp8 is not None:
        line["decode_fp8_kv"] = fp8
    if args.only == "all":
        print("bench: decode sweep", file=sys.stderr, flush=True)
        line["decode_sweep"] = bench_decode_sweep(max(5, args.steps // 2))
        print("bench: cascade prefill", file=sys.stderr, flush=True)
        line["cascade"] = bench_cascade(max(5, args.steps // 2))
        print("bench: cache writes and page-table build", file=sys.stderr, flush=True)
        line["pool"] = bench_pool(max(5, args.steps // 2))
        print("bench: merge_state", file=sys.stderr, flush=True)
        line["merge_state"] = bench_merge_state(max(5, args.steps // 2), flush)
    if not args.no_cpu_baseline and args.only == "all":
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(pre, dec, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
