#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM:
  1. batched paged GQA decode (bf16, B 64, Hq 32, Hkv 8, D 128, page 16,
     kv_len uniform in [512, 4096], pages scattered over a 300k-page pool):
     split-KV kernel + log-sum-exp combine;
  2. ragged causal prefill (bf16, B 8, L uniform in [1024, 4096], Hq 64,
     Hkv 8, D 128) packed by cu_seqlens;
  3. chunked prefill over a paged cache with a shared prefix (bf16, 16
     requests x 512-token chunks on 8192 cached tokens, Hq = Hkv = 16, D 256).

The headline value is decode KV throughput (algorithmic K+V bytes / decode
call time, GB/s); prefill TFLOPS (algorithmic causal flops / call time) is
reported beside it.  Before each timed segment a 1 GiB scratch buffer is
read (outside the segment's event pair) so every call starts with the inputs
in HBM but not in the MALL or the L2s.  Call times come from one event
pair per segment of the timed steps (mean, median and minimum); per-kernel
durations (the roofline figures) from a second pass in which the library
records HIP events around each of its launches on the launch stream.  Also
reported: the decode workload over an E4M3 (fp8) copy of its cache and
with the rotary position embedding, the
chunked workload through the shared-prefix cascade, the launch-bound fp32
single-sequence decode and the 1K-32K single-sequence
causal prefill sweep.  The CPU oracle is timed on the host cores beside
each workload (the whole decode workloads; every n-th query row of the
prefill workloads, with the exact flops of those rows), as a reported
baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-sweep] [--no-flush]
                       [--no-cpu-baseline] [--no-cascade] [--no-fp8] [--no-rope]
                       [--no-window] [--no-shapes] [--sweep-lengths L,...]
                       [--calibrate-copy MIB] [--only sweep|single]
Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
METRIC = "decode KV GB/s (% HBM peak); causal prefill TFLOPS (% bf16 MFMA peak)"


def per_launch(k, kind):
    """Mean ms per launch of `kind` from timing_end(), None when it never ran."""
    ms, n = k[kind]
    return round(ms / n, 5) if n else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-sweep", action="store_true", help="skip the 1K-32K single-sequence sweep")
    ap.add_argument("--no-flush", action="store_true",
                    help="do not read a 1 GiB scratch buffer before each timed segment")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cascade", action="store_true",
                    help="skip the shared-prefix cascade timing (its kernels share a name with "
                         "the direct paged prefill, so profiles of the latter skip it)")
    ap.add_argument("--no-fp8", action="store_true", help="skip the E4M3-cache decode timing")
    ap.add_argument("--no-rope", action="store_true", help="skip the rotary-embedding decode timing")
    ap.add_argument("--no-shapes", action="store_true",
                    help="skip the single 32K-request decode and the 64-token-page decode")
    ap.add_argument("--no-window", action="store_true",
                    help="skip the sliding-window decode and prefill timings")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="seconds of CPU-oracle work on the decode workload")
    ap.add_argument("--only", choices=("sweep", "single"), default=None,
                    help="profiling aid: run only the 1K-32K prefill sweep or only the fp32 "
                         "single-sequence decode (their kernels share names with other parts)")
    ap.add_argument("--sweep-lengths", default=None,
                    help="comma-separated subset of 1024,4096,16384,32768 for the sweep")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="finish with three plain device-to-device copies of MIB MiB, the "
                         "reference for HBM byte counters read under a profiler")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the kernels shard by request or head with no exchange; this benchmark measures one GPU)", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_qk_online_amd as A
    import workloads

    dev = torch.device("cuda:0")
    A.load_library()
    lengths = SWEEP_LENGTHS if args.sweep_lengths is None else tuple(
        int(x) for x in args.sweep_lengths.split(","))
    if any(L not in SWEEP_LENGTHS for L in lengths):
        print(f"--sweep-lengths takes values from {SWEEP_LENGTHS}", file=sys.stderr)
        sys.exit(2)
    if args.only is not None:
        # Profiling aid: one part on its own, one JSON line with its figures.
        if args.only == "single":
            part = bench_single(A, dev, args.steps)
        else:
            part = bench_sweep(A, dev, workloads.make_config(4), lengths, args.steps,
                               lambda: None)
        print(json.dumps({"only": args.only, "steps": args.steps, args.only: part}), flush=True)
        return

    # ---------------------------------------------------------------- inputs
    log("bench: generating inputs")
    dec = workloads.make_config(2)
    d_kp, d_vp = dec.pools(dev)
    d_q, d_table, d_lens = dec.q.to(dev), dec.page_table.to(dev), dec.kv_lens.to(dev)
    d_out = torch.empty_like(d_q)
    d_lse = torch.empty((dec.B, dec.Hq), dtype=torch.float32, device=dev)
    ws_bytes = A.decode_paged_workspace_size(dec.dtype, dec.B, dec.Hq, dec.Hkv, dec.D, dec.page_size,
                                             dec.max_kv_len, 0)
    d_ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)   # zero on first use

    pre = workloads.make_config(3)
    p_q, p_k, p_v = pre.q.to(dev), pre.k.to(dev), pre.v.to(dev)
    p_cq, p_ck = pre.cu_seqlens_q.to(dev), pre.cu_seqlens_k.to(dev)
    p_out = torch.empty_like(p_q)
    p_lse = torch.empty(p_q.shape[:2], dtype=torch.float32, device=dev)

    pg = workloads.make_config(5)
    g_q, g_cq = pg.q.to(dev), pg.cu_seqlens_q.to(dev)
    g_kp, g_vp = pg.pools(dev)
    g_table, g_lens = pg.page_table.to(dev), pg.kv_lens.to(dev)
    g_out = torch.empty_like(g_q)
    g_lse = torch.empty(g_q.shape[:2], dtype=torch.float32, device=dev)

    def decode():
        A.decode_paged(d_q, d_kp, d_vp, d_table, d_lens, scale=dec.scale, max_kv_len=dec.max_kv_len,
                       out=d_out, lse=d_lse, workspace=d_ws)

    def prefill():
        A.prefill_varlen(p_q, p_k, p_v, p_cq, p_ck, pre.max_seqlen_q, pre.max_seqlen_k, causal=True,
                         scale=pre.scale, out=p_out, lse=p_lse)

    def paged():
        A.prefill_paged(g_q, g_cq, g_kp, g_vp, g_table, g_lens, pg.max_seqlen_q, pg.max_kv_len,
                        causal=True, scale=pg.scale, out=g_out, lse=g_lse)

    # Before each timed segment (outside its event pair) a 1 GiB scratch buffer
    # is read, which evicts the inputs from the 256 MB MALL and the L2s and
    # leaves clean lines behind (a write would leave dirty ones whose
    # write-back then competes with the timed call).
    scratch = None if args.no_flush else torch.ones(1 << 28, dtype=torch.int32, device=dev)

    def flush():
        if scratch is not None:
            scratch.sum()

    stream = torch.cuda.current_stream(dev)
    log("bench: warmup")
    for _ in range(args.warmup):
        decode(); prefill(); paged()
    torch.cuda.synchronize()

    # ------------------------------------------------------------ timed steps
    # Pass 1 (the reported numbers): K steps bracketed by synchronisation, one
    # event pair per hot-path segment, no other instrumentation.
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_end = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        for j, seg in enumerate((decode, prefill, paged)):
            flush()
            ev[i][j].record(stream)
            seg()
            ev_end[i][j].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    log("bench: timed", K, "steps in", t1 - t0, "s")
    # Pass 2 (roofline): the same steps again with the library bracketing each
    # of its kernel launches by HIP events on the launch stream.
    A.timing_begin(8 * K + 16)
    for i in range(K):
        for seg in (decode, prefill, paged):
            flush()
            seg()
    kt = A.timing_end()

    seg_ms = [sorted(ev[i][j].elapsed_time(ev_end[i][j]) for i in range(K)) for j in range(3)]

    def stats(ms):
        return {"mean": round(sum(ms) / len(ms), 5), "median": round(ms[len(ms) // 2], 5),
                "min": round(ms[0], 5)}
    ms_decode, ms_prefill, ms_paged = (sum(x) / len(x) for x in seg_ms)

    def avg(kind):
        ms, n = kt.get(kind, (0.0, 0))
        return ms / n if n else None

    kv_bytes = dec.kv_bytes()
    pre_flops = pre.flops()
    pg_flops = pg.flops()
    split_ms = avg("decode_split")
    prefill_ms = avg("prefill")
    paged_ms = avg("prefill_paged")
    decode_gbs = kv_bytes / (ms_decode * 1e-3) / 1e9

    def roofline_hbm(nbytes, ms, kernel):
        a = nbytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4), "traffic": measured_traffic(kernel)}

    def roofline_mfma(flops, ms, kernel):
        a = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(a, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(a / BF16_PEAK_TFLOPS, 4), "traffic": measured_traffic(kernel)}

    res = {
        "metric": METRIC,
        "value": round(decode_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1e3 / K, 4),
        # ms_per_step is wall time per step and includes the three cache
        # flushes; this is the hot path alone (mean call times, flushes out).
        "hot_path_ms_per_step": round(ms_decode + ms_prefill + ms_paged, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workloads.CONFIG_NAMES[2], "B": dec.B, "Hq": dec.Hq, "Hkv": dec.Hkv,
                   "D": dec.D, "page_size": dec.page_size, "pool_pages": dec.num_pages,
                   "sum_kv_len": int(dec.kv_lens.sum()), "kv_bytes": kv_bytes,
                   "step": "paged decode + ragged causal prefill + chunked paged prefill"},
        "cache_flush_bytes": 0 if scratch is None else scratch.numel() * 4,
        "decode": {"call_ms": round(ms_decode, 5), "call_ms_stats": stats(seg_ms[0]),
                   "split_kernel_ms": round(split_ms, 5),
                   "combine_kernel_ms": None if avg("decode_combine") is None
                   else round(avg("decode_combine"), 5),
                   "frac_of_hbm_peak": round(decode_gbs / HBM_PEAK_GBS, 4)},
        "roofline": roofline_hbm(kv_bytes, split_ms, "decode_split"),
        "prefill": {
            "metric": "causal prefill TFLOPS", "unit": "TFLOP/s",
            "value": round(pre_flops / (ms_prefill * 1e-3) / 1e12, 2),
            "workload": workloads.CONFIG_NAMES[3], "flops": pre_flops,
            "call_ms": round(ms_prefill, 4), "call_ms_stats": stats(seg_ms[1]),
            "kernel_ms": round(prefill_ms, 4),
            "roofline": roofline_mfma(pre_flops, prefill_ms, "prefill"),
        },
        "prefill_paged": {
            "metric": "chunked paged prefill TFLOPS", "unit": "TFLOP/s",
            "value": round(pg_flops / (ms_paged * 1e-3) / 1e12, 2),
            "workload": workloads.CONFIG_NAMES[5], "flops": pg_flops,
            "call_ms": round(ms_paged, 4), "call_ms_stats": stats(seg_ms[2]),
            "kernel_ms": round(paged_ms, 4),
            "roofline": roofline_mfma(pg_flops, paged_ms, "prefill_paged"),
        },
    }

    # The decode workload over an E4M3 copy of its cache (one scale per K / V
    # tensor): half the bytes through the same schedule.
    if not args.no_fp8:
        f_kp, f_vp, f_ks, f_vs = dec.fp8_pools(dev)
        f_bytes = dec.fp8_kv_bytes()

        def decode_fp8():
            A.decode_paged_fp8(d_q, f_kp, f_vp, d_table, d_lens, f_ks, f_vs, scale=dec.scale,
                               max_kv_len=dec.max_kv_len, out=d_out, lse=d_lse, workspace=d_ws)
        for _ in range(3):
            decode_fp8()
        torch.cuda.synchronize()
        for i in range(K):
            flush()
            ev[i][0].record(stream)
            decode_fp8()
            ev_end[i][0].record(stream)
        torch.cuda.synchronize()
        f_ms = sorted(ev[i][0].elapsed_time(ev_end[i][0]) for i in range(K))
        A.timing_begin(2 * K + 4)
        for i in range(K):
            flush()
            decode_fp8()
        kf = A.timing_end()
        f_mean = sum(f_ms) / K
        f_split = kf["decode_split"][0] / kf["decode_split"][1]
        res["decode_fp8"] = {
            "metric": "decode KV GB/s over an E4M3 cache", "unit": "GB/s",
            "value": round(f_bytes / (f_mean * 1e-3) / 1e9, 1), "kv_bytes": f_bytes,
            "call_ms": round(f_mean, 5), "call_ms_stats": stats(f_ms),
            "split_kernel_ms": round(f_split, 5),
            "combine_kernel_ms": per_launch(kf, "decode_combine"),
            "speedup_vs_bf16_call": round(ms_decode / f_mean, 4),
            "roofline": roofline_hbm(f_bytes, f_split, "decode_fp8")}
        log("bench: fp8 decode", res["decode_fp8"])
        del f_kp, f_vp

    # The decode workload with the rotary position embedding (theta 10000)
    # applied to the query and to every cached key inside the kernel: the
    # same bytes as the plain decode, more arithmetic per page.
    if not args.no_rope:
        def decode_rope():
            A.decode_paged(d_q, d_kp, d_vp, d_table, d_lens, scale=dec.scale,
                           max_kv_len=dec.max_kv_len, out=d_out, lse=d_lse, workspace=d_ws,
                           rope_theta=10000.0)
        for _ in range(3):
            decode_rope()
        torch.cuda.synchronize()
        for i in range(K):
            flush()
            ev[i][0].record(stream)
            decode_rope()
            ev_end[i][0].record(stream)
        torch.cuda.synchronize()
        r_ms = sorted(ev[i][0].elapsed_time(ev_end[i][0]) for i in range(K))
        A.timing_begin(2 * K + 4)
        for i in range(K):
            flush()
            decode_rope()
        kr = A.timing_end()
        r_mean = sum(r_ms) / K
        r_split = kr["decode_split"][0] / kr["decode_split"][1]
        res["decode_rope"] = {
            "metric": "decode KV GB/s with the rotary embedding", "unit": "GB/s",
            "value": round(kv_bytes / (r_mean * 1e-3) / 1e9, 1), "rope_theta": 10000.0,
            "call_ms": round(r_mean, 5), "call_ms_stats": stats(r_ms),
            "split_kernel_ms": round(r_split, 5),
            "combine_kernel_ms": per_launch(kr, "decode_combine"),
            "slowdown_vs_plain_call": round(r_mean / ms_decode, 4),
            "roofline": roofline_hbm(kv_bytes, r_split, "decode_rope")}
        log("bench: rope decode", res["decode_rope"])

    # Sliding windows on the same workloads: the decode workload with a
    # 1024-key window (pages before each window never read), the ragged causal
    # prefill with a 1024-key window, and the ragged workload non-causal with
    # the band window (512, 256).  Rates count only what the window leaves
    # visible: K+V bytes of the keys in each window, flops of the visible pairs.
    def timed(fn, kinds):
        """K calls after a flush each: sorted call times (event pairs) and the
        mean duration of each kernel kind (the library's launch events)."""
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        for i in range(K):
            flush()
            ev[i][0].record(stream)
            fn()
            ev_end[i][0].record(stream)
        torch.cuda.synchronize()
        ms = sorted(ev[i][0].elapsed_time(ev_end[i][0]) for i in range(K))
        A.timing_begin(2 * K + 4)
        for i in range(K):
            flush()
            fn()
        kw = A.timing_end()
        return ms, {k: kw[k][0] / kw[k][1] for k in kinds if kw[k][1]}

    if not args.no_window:
        wdec = 1024
        w_bytes = 2 * dec.Hkv * dec.D * dec.dtype.itemsize * sum(
            min(int(x), wdec + 1) for x in dec.kv_lens.tolist())
        ms, kk = timed(lambda: A.decode_paged(d_q, d_kp, d_vp, d_table, d_lens, scale=dec.scale,
                                              max_kv_len=dec.max_kv_len, out=d_out, lse=d_lse,
                                              workspace=d_ws, window_left=wdec),
                       ("decode_split", "decode_combine"))
        mean = sum(ms) / K
        a = w_bytes / (kk["decode_split"] * 1e-3) / 1e9
        windows = {"decode": {
            "workload": workloads.CONFIG_NAMES[2], "window_left": wdec, "kv_bytes_visible": w_bytes,
            "value": round(w_bytes / (mean * 1e-3) / 1e9, 1), "unit": "GB/s",
            "call_ms": round(mean, 5), "call_ms_stats": stats(ms),
            "split_kernel_ms": round(kk["decode_split"], 5),
            "roofline": {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(a / HBM_PEAK_GBS, 4), "traffic": None}}}
        for name, causal, left, right in (("prefill_causal_window_1024", True, 1024, -1),
                                          ("prefill_band_512_256", False, 512, 256)):
            fl = 4 * pre.D * pre.Hq * visible_pairs(pre.lens_q, pre.lens_k, causal, left, right)
            ms, kk = timed(lambda: A.prefill_varlen(p_q, p_k, p_v, p_cq, p_ck, pre.max_seqlen_q,
                                                    pre.max_seqlen_k, causal=causal, scale=pre.scale,
                                                    out=p_out, lse=p_lse, window_left=left,
                                                    window_right=right), ("prefill",))
            mean = sum(ms) / K
            a = fl / (kk["prefill"] * 1e-3) / 1e12
            windows[name] = {
                "workload": workloads.CONFIG_NAMES[3], "causal": causal, "window_left": left,
                "window_right": right, "flops_visible": fl,
                "value": round(fl / (mean * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                "call_ms": round(mean, 4), "call_ms_stats": stats(ms),
                "kernel_ms": round(kk["prefill"], 4),
                "roofline": {"bound": "mfma", "achieved": round(a, 1), "peak": BF16_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(a / BF16_PEAK_TFLOPS, 4),
                             "traffic": None}}
        res["windows"] = windows
        log("bench: windows", windows)

    # Two more decode shapes of the same model (Hq 32, Hkv 8, D 128, bf16): one
    # 32768-token request (every head group split over all runs, merged by
    # the segment-parallel merge), and the decode workload's lengths over a
    # cache of 64-token pages.
    if not args.no_shapes:
        shapes = {}
        for name, kw in (("b1_kv32768_p16", dict(B=1, page_size=16, kv_lens=[32768], seed=21)),
                         ("b64_kv512-4096_p64", dict(B=dec.B, page_size=64, kv_lens=dec.kv_lens,
                                                     seed=22))):
            c = workloads.make_decode(Hq=dec.Hq, Hkv=dec.Hkv, D=dec.D, dtype=dec.dtype, **kw)
            s_kp, s_vp = c.pools(dev)
            s_q, s_t, s_l = c.q.to(dev), c.page_table.to(dev), c.kv_lens.to(dev)
            s_out, s_lse = torch.empty_like(s_q), torch.empty(c.B, c.Hq, device=dev)
            s_ws = torch.empty(max(1, A.decode_paged_workspace_size(c.dtype, c.B, c.Hq, c.Hkv, c.D,
                                                                    c.page_size, c.max_kv_len, 0)),
                               dtype=torch.uint8, device=dev)
            ms, kk = timed(lambda: A.decode_paged(s_q, s_kp, s_vp, s_t, s_l, scale=c.scale,
                                                  max_kv_len=c.max_kv_len, out=s_out, lse=s_lse,
                                                  workspace=s_ws), ("decode_split", "decode_combine"))
            nb = c.kv_bytes()
            mean = sum(ms) / K
            a = nb / (kk["decode_split"] * 1e-3) / 1e9
            shapes[name] = {
                "kv_bytes": nb, "value": round(nb / (mean * 1e-3) / 1e9, 1), "unit": "GB/s",
                "call_ms": round(mean, 5), "call_ms_stats": stats(ms),
                "split_kernel_ms": round(kk["decode_split"], 5),
                "combine_kernel_ms": round(kk["decode_combine"], 5) if "decode_combine" in kk else None,
                "roofline": {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(a / HBM_PEAK_GBS, 4), "traffic": None}}
            del s_kp, s_vp
        res["decode_shapes"] = shapes
        log("bench: decode shapes", shapes)

    # The chunked workload again through the shared-prefix cascade: one pass
    # of every query row over the 4096 shared tokens, then each request over
    # its own keys with the merge fused into the store.  Same flops as the
    # direct call (the work is split, not skipped).
    if not args.no_cascade:
        prefix_len = pg.shared_pages * pg.page_size
        c_ws = torch.empty(A.prefill_paged_cascade_workspace_size(pg.dtype, g_q.shape[0], pg.Hq,
                                                                  pg.D),
                           dtype=torch.uint8, device=dev)

        def cascade():
            A.prefill_paged_cascade(g_q, g_cq, g_kp, g_vp, g_table, g_lens, pg.max_seqlen_q,
                                    pg.max_kv_len, prefix_len, causal=True, scale=pg.scale,
                                    out=g_out, lse=g_lse, workspace=c_ws)
        for _ in range(2):
            cascade()
        torch.cuda.synchronize()
        for i in range(K):
            flush()
            ev[i][0].record(stream)
            cascade()
            ev_end[i][0].record(stream)
        torch.cuda.synchronize()
        c_ms = sorted(ev[i][0].elapsed_time(ev_end[i][0]) for i in range(K))
        A.timing_begin(2 * K + 4)
        for i in range(K):
            flush()
            cascade()
        kc = A.timing_end()
        c_mean = sum(c_ms) / K
        res["prefill_paged"]["cascade"] = {
            "shared_prefix_len": prefix_len,
            "value": round(pg_flops / (c_mean * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "call_ms": round(c_mean, 4), "call_ms_stats": stats(c_ms),
            "prefix_kernel_ms": round(kc["cascade_prefix"][0] / kc["cascade_prefix"][1], 4),
            "suffix_kernel_ms": round(kc["cascade_suffix"][0] / kc["cascade_suffix"][1], 4),
            "speedup_vs_direct": round(ms_paged / c_mean, 4)}
        log("bench: cascade", res["prefill_paged"]["cascade"])
        del c_ws

    res["decode_fp32_single"] = bench_single(A, dev, K)

    if not args.no_sweep:
        del p_q, p_k, p_v, p_out, p_lse
        long = workloads.make_config(4)
        res["prefill_sweep"] = bench_sweep(A, dev, long, lengths, K, flush)

    if not args.no_cpu_baseline:
        # The oracle as it stands, on the host cores, after the GPU timing:
        # one leg per workload (and per sweep length), each placed beside
        # that workload's GPU figures.
        threads, tinfo = cpu_threads()
        torch.set_num_threads(threads)
        res["cpu_baseline"] = cpu_baseline(dec, args.cpu_seconds, threads)
        log("bench: cpu baseline (oracle), single fp32 decode")
        res["decode_fp32_single"]["cpu_baseline"] = cpu_single(workloads.make_config(1), threads)
        log("bench: cpu baseline (oracle), ragged prefill")
        res["prefill"]["cpu_baseline"] = cpu_prefill(pre, CPU_STRIDE["prefill"], threads)
        log("bench: cpu baseline (oracle), chunked paged prefill")
        res["prefill_paged"]["cpu_baseline"] = cpu_prefill(pg, CPU_STRIDE["prefill_paged"], threads,
                                                           paged=True)
        if not args.no_sweep:
            for L in lengths:
                log("bench: cpu baseline (oracle), sweep", L)
                res["prefill_sweep"]["by_length"][str(L)]["cpu_baseline"] = cpu_prefill(
                    long.prefix(L), CPU_STRIDE["sweep"][L], threads)
        res["cpu_host"] = dict(tinfo, threads=threads, cpu_model=cpu_model())

    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["calibrate_copy_bytes"] = n

    print(json.dumps(res), flush=True)


def bench_single(A, dev, K):
    """The launch-bound fp32 single-sequence decode: eager call times and the
    per-call share of a HIP graph of 20 calls."""
    import torch
    import workloads
    stream = torch.cuda.current_stream(dev)
    # Single-sequence fp32 decode (1 query token, 4 heads, head_dim 64, 256
    # contiguous keys as an identity-paged NHD view): launch-latency bound.
    one = workloads.make_config(1)
    o_kp, o_vp = one.pools(dev)
    o_q, o_t, o_l = one.q.to(dev), one.page_table.to(dev), one.kv_lens.to(dev)

    o_ws = torch.empty(max(1, A.decode_paged_workspace_size(one.dtype, one.B, one.Hq, one.Hkv, one.D,
                                                            one.page_size, one.max_kv_len, 0)),
                       dtype=torch.uint8, device=dev)

    def single():
        A.decode_paged(o_q, o_kp, o_vp, o_t, o_l, scale=one.scale, max_kv_len=one.max_kv_len,
                       workspace=o_ws)
    for _ in range(5):
        single()
    torch.cuda.synchronize()
    e0 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    e1 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for i in range(K):
        e0[i].record(stream)
        single()
        e1[i].record(stream)
    torch.cuda.synchronize()
    one_ms = sorted(e0[i].elapsed_time(e1[i]) for i in range(K))
    # Kernel durations (the library's launch events): the split kernel and
    # the combine of its two partial states.
    A.timing_begin(2 * K + 4)
    for i in range(K):
        single()
    kk = A.timing_end()
    split_ms = kk["decode_split"][0] / kk["decode_split"][1]
    comb_ms = kk["decode_combine"][0] / kk["decode_combine"][1] if kk["decode_combine"][1] else None
    # The same call captured 20 times back to back in one HIP graph (static
    # buffers) and replayed: the per-call share of a replay, as when the
    # decode of many layers is captured together.
    NG = 20
    g_out, g_lse = torch.empty_like(o_q), torch.empty(one.B, one.Hq, device=dev)

    def single_static():
        A.decode_paged(o_q, o_kp, o_vp, o_t, o_l, scale=one.scale, max_kv_len=one.max_kv_len,
                       out=g_out, lse=g_lse)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        single_static()
    stream.wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(NG):
            single_static()
    graph.replay()
    torch.cuda.synchronize()
    for i in range(K):
        e0[i].record(stream)
        graph.replay()
        e1[i].record(stream)
    torch.cuda.synchronize()
    rep_ms = sorted(e0[i].elapsed_time(e1[i]) / NG for i in range(K))
    return {
        "workload": workloads.CONFIG_NAMES[1], "kv_bytes": one.kv_bytes(),
        "call_us_median": round(one_ms[K // 2] * 1e3, 2), "call_us_min": round(one_ms[0] * 1e3, 2),
        "GBs_at_median": round(one.kv_bytes() / (one_ms[K // 2] * 1e-3) / 1e9, 2),
        "graph_us_per_call_median": round(rep_ms[K // 2] * 1e3, 2),
        "graph_us_per_call_min": round(rep_ms[0] * 1e3, 2),
        "split_kernel_us": round(split_ms * 1e3, 3),
        "combine_kernel_us": None if comb_ms is None else round(comb_ms * 1e3, 3),
        "roofline": {"bound": "hbm", "achieved": round(one.kv_bytes() / (split_ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(one.kv_bytes() / (split_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
                     "traffic": None},
        "note": "launch-latency bound (512 KiB of KV). Eager: one event pair around one call "
                "(host overhead included). Graph: 20 calls captured in one graph, replay time / 20"}


SWEEP_LENGTHS = (1024, 4096, 16384, 32768)


def bench_sweep(A, dev, long, lengths, K, flush):
    """Single-sequence causal prefill over the first L tokens of the 32K
    workload: mean kernel duration (the library's launch events) per length."""
    import torch
    import workloads
    q, k, v = long.q.to(dev), long.k.to(dev), long.v.to(dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    sweep = {}
    for L in lengths:
        cu = torch.tensor([0, L], dtype=torch.int32, device=dev)
        fl = workloads.prefill_flops([L], [L], long.Hq, long.D, True)
        reps = max(3, min(K, int(2e12 / fl * 20)))

        def call():
            A.prefill_varlen(q[:L], k[:L], v[:L], cu, cu, L, L, causal=True, scale=long.scale,
                             out=out[:L], lse=lse[:L])
        for _ in range(2):
            call()
        torch.cuda.synchronize()
        A.timing_begin(reps + 4)
        for _ in range(reps):
            flush()
            call()
        kk = A.timing_end()
        ms = kk["prefill"][0] / kk["prefill"][1]
        sweep[str(L)] = {"flops": fl, "launches": reps, "kernel_ms": round(ms, 4),
                         "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                         "frac": round(fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
        log("bench: sweep", L, sweep[str(L)])
    return {"workload": workloads.CONFIG_NAMES[4], "by_length": sweep}


# Measured HBM traffic per launch (FETCH_SIZE + WRITE_SIZE under rocprofv3,
# scaled by what the same counters read for a plain copy of known size) is
# kept in a profile summary together with the SHA-256 of the sources it was
# measured on; it is reported only while those sources are unchanged.
TRAFFIC_FILES = {
    "decode_split": "profiles/traffic__decode_split__paged_decode_b64_hq32_hkv8_d128.md",
    "decode_fp8": "profiles/traffic__decode_split_fp8__paged_decode_e4m3_b64_hq32_hkv8_d128.md",
    "decode_rope": "profiles/traffic__decode_split_rope__paged_decode_rope_b64_hq32_hkv8_d128.md",
    "prefill": "profiles/traffic__prefill__ragged_causal_b8_hq64_hkv8_d128.md",
    "prefill_paged": "profiles/traffic__prefill_paged__chunked_b16_q512_kv8704_h16_d256.md",
}
KERNEL_SOURCES = {
    "decode_split": ["decode.hip"],
    "decode_fp8": ["decode.hip"],
    "decode_rope": ["decode.hip"],
    "prefill": ["prefill.hip"],
    "prefill_paged": ["prefill256.hip"],     # the chunked workload has head_dim 256
}


def _code_only(text):
    """Source text without comments and blank space, so that a comment edit
    does not count as a kernel change."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(kind):
    """SHA-256 over the code (comments dropped) of the sources that build one
    kernel: its .hip file plus the shared headers and the host-side launch code."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_qk_online_amd", "csrc")
    for name in KERNEL_SOURCES[kind] + ["common.h", "launch.h", "api.cpp"]:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()


def measured_traffic(kind):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, TRAFFIC_FILES[kind])
    try:
        text = open(path).read()
    except OSError:
        return None
    start = text.find("```json")
    if start < 0:
        return None
    rec = json.loads(text[start + 7:text.index("```", start + 7)])
    if rec.get("source_sha256") != source_digest(kind):
        return None
    return int(rec["hbm_bytes_per_launch"])


def visible_pairs(lens_q, lens_k, causal, left=-1, right=-1):
    """(query, key) pairs a windowed attention computes: query i of a sequence
    sees keys i + (Lk - Lq) - left .. i + (Lk - Lq) + right within 0 .. Lk - 1
    (-1: that side open; causal is the right bound 0)."""
    import torch
    shift = 0 if causal else right
    tot = 0
    for lq, lk in zip(lens_q, lens_k):
        i = torch.arange(lq, dtype=torch.int64)
        hi = torch.full_like(i, lk - 1)
        if shift >= 0:
            hi = torch.minimum(hi, i + (lk - lq) + shift)
        lo = torch.zeros_like(i)
        if left >= 0:
            lo = torch.maximum(lo, i + (lk - lq) - left)
        tot += int((hi - lo + 1).clamp(min=0).sum())
    return tot


def cpu_threads():
    """Threads for the CPU oracle: the CPUs this process may run on (its
    affinity mask), bounded by the cgroup CPU quota and by OMP_NUM_THREADS
    when either is set -- a container or a scheduler that runs one job per
    GPU gives each job a share of the host (os.cpu_count() reports the whole
    machine).  Returns (threads, details)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    info = {"os_cpu_count": os.cpu_count(), "affinity_cpus": n}
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()
        if quota != "max":
            q = max(1, int(quota) // int(period))
            info["cgroup_quota_cpus"] = q
            n = min(n, q)
    except (OSError, ValueError):
        pass
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        info["OMP_NUM_THREADS"] = int(omp)
        n = min(n, int(omp))
    return max(1, n), info


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(dec, seconds, threads):
    """The float64 oracle over the whole decode workload on the host cores,
    repeated until at least ``seconds`` have passed; GB/s of algorithmic KV bytes."""
    import torch
    import oracle
    log("bench: cpu baseline (oracle), decode")
    # The oracle only reads referenced pages, so the pool is left unfilled elsewhere.
    shape = (dec.num_pages, dec.page_size, dec.Hkv, dec.D)
    kp = torch.empty(shape, dtype=dec.dtype)
    vp = torch.empty(shape, dtype=dec.dtype)
    kp.view(-1, dec.Hkv, dec.D).index_copy_(0, dec.slot_index, dec.k_tok)
    vp.view(-1, dec.Hkv, dec.D).index_copy_(0, dec.slot_index, dec.v_tok)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.ref_decode_paged(dec.q, kp, vp, dec.page_table, dec.kv_lens, dec.scale)
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(dec.kv_bytes() * reps / dt / 1e9, 3), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"whole workload ({dec.B} requests) x {reps} repetitions, {dt:.1f} s, "
                      f"float64 torch on CPU",
            "ms_per_call": round(dt * 1e3 / reps, 2)}


def sampled_pairs(lens_q, lens_k, rows, causal):
    """Visible (query, key) pairs per head of the given global query rows
    (causal: bottom-right aligned), summed."""
    import bisect
    cu = [0]
    for L in lens_q:
        cu.append(cu[-1] + int(L))
    tot = 0
    for r in rows:
        b = bisect.bisect_right(cu, r) - 1
        i, lq, lk = r - cu[b], int(lens_q[b]), int(lens_k[b])
        tot += min(max(i + lk - lq + 1, 0), lk) if causal else lk
    return tot


def cpu_prefill(case, stride, threads, paged=False):
    """The float64 oracle on every ``stride``-th query row (all heads) of a
    prefill workload: effective TFLOP/s over the algorithmic flops of those rows."""
    import torch
    import oracle
    Tq = case.q.shape[0]
    rows = torch.arange(0, Tq, stride)
    lens_k = case.kv_lens.tolist() if paged else case.lens_k
    pairs = sampled_pairs(case.lens_q, lens_k, rows.tolist(), case.causal)
    flops = 4 * case.D * case.Hq * pairs
    t0 = time.perf_counter()
    if paged:
        oracle.ref_prefill_paged(case.q, case.cu_seqlens_q, case.pool_k, case.pool_v,
                                 case.page_table, case.kv_lens, case.causal, case.scale, rows=rows)
    else:
        oracle.ref_prefill_varlen(case.q, case.k, case.v, case.cu_seqlens_q, case.cu_seqlens_k,
                                  case.causal, case.scale, rows=rows)
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{rows.numel()} of {Tq} query rows (every {stride}th row, all {case.Hq} "
                      f"heads): {pairs} visible pairs per head, {flops} algorithmic flops, "
                      f"{dt:.2f} s, float64 torch on CPU",
            "ms": round(dt * 1e3, 1), "flops": flops}


def cpu_single(one, threads, seconds=1.0):
    """The float64 oracle over the single-sequence fp32 decode, repeated for
    at least ``seconds``."""
    import oracle
    kp, vp = one.pools()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.ref_decode_paged(one.q, kp, vp, one.page_table, one.kv_lens, one.scale)
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(one.kv_bytes() * reps / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"whole workload x {reps} repetitions, {dt:.2f} s, float64 torch on CPU",
            "us_per_call": round(dt * 1e6 / reps, 1)}


# Row strides of the CPU samples: each leg is a few seconds of float64 work
# on 16 host threads.
CPU_STRIDE = {"prefill": 16, "prefill_paged": 16,
              "sweep": {1024: 1, 4096: 16, 16384: 64, 32768: 128}}


if __name__ == "__main__":
    main()
