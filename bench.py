#!/usr/bin/env python3
"""Benchmark of the fused LM-head + exact Gumbel-Max sampler on one MI355X.

One step = one sampler call (LM-head contraction, temperature scaling,
Gumbel perturbation, per-tile (max, argmax), merge) over one batch of the
Llama-3-8B-shaped LM head (D = 4096, V = 128256, bf16), with the inputs
already resident in device memory and a fresh (seed, step) per step.  The
headline step is fs_sample_packed at B = 32: W is re-tiled once into the
kernels' fragment order (fs_pack_weights, as at model load, outside the
timed region); every step reads the same bytes and does the same work as
fs_sample on the row-major W, whose figures the line carries beside it
("row_major"; --no-packed makes row-major the headline).  The same line
carries the B = 1 .. 256 sweep, the
unfused baseline (logits and probabilities through device memory) timed the
same way, the grouped (hierarchical) sampler over 1 and 8 vocabulary groups
(all groups in one launch, and one launch per group), the online sampler with
early finalisation (8 vocabulary chunks), the packed (fragment-order) weight
path beside each row-major figure, the Qwen3-shaped, large-batch and
vocabulary-shard heads, the fused kernel's roofline fraction and the CPU
oracle's rate.  For context it also times the bf16 GEMM alone through
torch.matmul (ROCm's BLAS library) at the headline batch, at B = 256 and on
the large-batch head at B = 512.

Prints ONE JSON line on stdout.  Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--batch 32]
                  [--sweep 1,2,4,...] [--no-cpu-baseline] [--no-unfused]
                  [--no-grouped] [--no-online] [--no-packed] [--no-workloads]
                  [--no-gemm-context]
                  [--profile-pass]
--profile-pass runs a short fixed sequence for rocprofv3 (a few fused steps
plus a 1 GiB device copy used to calibrate the HBM byte counters) and exits.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused LM-head+sample µs/step & % roofline, B=1..256, D=4096, V=128256"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=32)
    ap.add_argument("--sweep", default="1,2,4,8,16,32,64,128,256")
    ap.add_argument("--sweep-steps", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unfused", action="store_true")
    ap.add_argument("--no-grouped", action="store_true")
    ap.add_argument("--no-gemm-context", action="store_true")
    ap.add_argument("--no-workloads", action="store_true")
    ap.add_argument("--no-online", action="store_true")
    ap.add_argument("--no-packed", action="store_true")
    ap.add_argument("--profile-pass", action="store_true")
    ap.add_argument("--profile-workload", default="llama3-8b-lm-head",
                    help="workload of --profile-pass (a name from lm_head_exact_amd.workloads)")
    return ap.parse_args()


def algorithmic_bytes(B, D, V):
    """Bytes the fused step must move: W and h read once, T read, one
    (id, score) pair written per row.  Per-tile partials are implementation
    traffic (8 bytes per row per tile, under 0.2 % here) and not counted."""
    return 2 * V * D + 2 * B * D + 4 * B + 8 * B


def flops(B, D, V):
    return 2 * B * V * D


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "fused_sample_llama3_b32_memory_counters.txt")


def kernel_sources_sha256():
    """Fingerprint of the sources the fused sampler kernels are compiled
    from: counters taken on other sources no longer describe the kernel that
    runs.  (Which configuration runs is checked by name, beside it; the
    configuration table, the merges, the unfused baseline and the host-side
    API live in other files.)"""
    import hashlib
    csrc = os.path.join(ROOT, "lm_head_exact_amd", "csrc")
    h = hashlib.sha256()
    for name in ("fs_device.hpp", "fs_internal.hpp", "fs_mma.hpp", "fs_sampler.hpp",
                 "fs_configs_small.hip", "fs_configs_lds.hip",
                 "fs_configs_dma_a.hip", "fs_configs_dma_b.hip", "fs_configs_dma_ntl.hip"):
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def measured_traffic(B, config):
    """HBM bytes per launch of the fused kernel (read + written) from the
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, calibrated against a
    copy of known size; None when absent, taken at another batch size, on
    another configuration or on different kernel sources."""
    try:
        kv = {}
        for line in open(TRAFFIC_PROFILE):
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
        if kv.get("kernel_sources_sha256") != kernel_sources_sha256():
            return None
        if int(kv.get("batch", -1)) != B or kv.get("config") != config:
            return None
        return int(float(kv["hbm_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def roofline_us(B, D, V):
    return max(algorithmic_bytes(B, D, V) / (HBM_PEAK_GBS * 1e3),
               flops(B, D, V) / (MFMA_BF16_PEAK_TFLOPS * 1e6))


def time_steps(torch, fn, steps, warmup, stream):
    """Warm up, then time `steps` calls between two events on `stream`;
    returns milliseconds per step."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        fn(warmup + i)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def step_percentiles(torch, fn, steps, warmup, stream):
    """Each of `steps` calls timed on its own (an event before and after it on
    `stream`); returns (p10, median, p90) in microseconds."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn(warmup + i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    d = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps))

    def q(f):
        return d[min(len(d) - 1, int(round(f * (len(d) - 1))))]
    return q(0.10), q(0.50), q(0.90)


def device_peaks(fsl, dev):
    """CU count and peak shader clock the HIP runtime reports (through the
    library), and the dense bf16 MFMA peak they imply: CUs x 4 SIMDs x one
    16x16x32 MFMA (8192 multiply-adds) per 16 clocks per SIMD x 2 FLOP x
    clock.  The roofline uses the published peaks; this is printed beside
    them."""
    cus, clock_khz = fsl.device_info(dev.index or 0)
    peak = cus * 4 * (8192 / 16) * 2 * clock_khz * 1e3 / 1e12
    return {"cus": cus, "clock_khz": clock_khz,
            "bf16_dense_tflops_from_clock": round(peak, 1),
            "bf16_dense_tflops_used": MFMA_BF16_PEAK_TFLOPS, "hbm_gbs_used": HBM_PEAK_GBS}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def measure_fused_kernel(torch, fsl, fn, steps, warmup):
    """Launch bracket of the fused kernel: HIP events the library records on
    the caller's stream right before and right after each fused-kernel launch
    (fs_profile_enable).  The bracket holds the kernel and its dispatch after
    the preceding work on the stream, not the tile merge that follows it;
    rocprofv3's kernel trace gives the kernel alone (a few microseconds
    less).  Returns (mean, min, max) in ms and the launch count."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    fsl.profile_enable(steps)
    for i in range(steps):
        fn(warmup + i)
    n, tot, lo, hi = fsl.profile_read()
    fsl.profile_enable(0)
    return tot / max(n, 1), lo, hi, n


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the sampler runs on one device; see the sharding notes in the design document)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import lm_head_exact_amd as fsl
    from lm_head_exact_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    wlk = wl.LLAMA3_8B
    D, V = wlk.D, wlk.V
    W = wl.make_w(wlk, dev)
    stream = torch.cuda.current_stream(dev)

    # W in fragment order (packed once, as at model load) for fs_sample_packed
    Wp = fsl.pack_weights(W) if not args.no_packed else None

    def make_step(B, unfused=False, packed=False):
        h = wl.make_h(wlk, B, dev)
        T = wl.make_temperature(wlk, B, dev)
        out = (torch.empty(B, dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.float32, device=dev))
        if unfused:
            ws = fsl.alloc_workspace(fsl.unfused_workspace_bytes(B, D, V), dev)
            call = fsl.sample_unfused
        else:
            ws = fsl.alloc_workspace(fsl.workspace_bytes(B, D, V), dev)
            call = fsl.sample

        def fn(i):
            seed, step = wlk.sampler_seed(i)
            if packed:
                fsl.sample_packed(h, Wp, V, T, seed, step, out=out, workspace=ws)
            else:
                call(h, W, T, seed, step, out=out, workspace=ws)
        return fn, (h, T, out, ws)

    if args.profile_pass:
        pw = wl.WORKLOADS[args.profile_workload]
        if pw is wlk:
            fn, keep = make_step(args.batch, packed=Wp is not None)
        else:  # another head: its own weights (packed unless --no-packed) and inputs
            del W, Wp
            Wx = wl.make_w(pw, dev)
            Wpx = fsl.pack_weights(Wx, pw.vocab_offset) if not args.no_packed else None
            hx, Tx = wl.make_h(pw, args.batch, dev), wl.make_temperature(pw, args.batch, dev)
            outx = (torch.empty(args.batch, dtype=torch.int32, device=dev),
                    torch.empty(args.batch, dtype=torch.float32, device=dev))
            wsx = fsl.alloc_workspace(fsl.workspace_bytes(args.batch, pw.D, pw.V), dev)

            def fn(i):
                seed, step = pw.sampler_seed(i)
                if Wpx is not None:
                    fsl.sample_packed(hx, Wpx, pw.V, Tx, seed, step, pw.vocab_offset, out=outx,
                                      workspace=wsx)
                else:
                    fsl.sample(hx, Wx, Tx, seed, step, pw.vocab_offset, out=outx, workspace=wsx)
        for i in range(5):
            fn(i)
        torch.cuda.synchronize()
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)          # 1 GiB read + 1 GiB write: counter calibration
        torch.cuda.synchronize()
        print(json.dumps({"profile_pass": True, "workload": args.profile_workload, "B": args.batch,
                          "copy_bytes": 1 << 30}))
        return

    B = args.batch
    headline_packed = Wp is not None
    fn, keep = make_step(B, packed=headline_packed)
    ms = time_steps(torch, fn, args.steps, args.warmup, stream)
    p10, p50, p90 = step_percentiles(torch, fn, max(args.steps, 100), args.warmup, stream)
    k_ms, k_lo, k_hi, k_n = measure_fused_kernel(torch, fsl, fn, args.steps, args.warmup)
    us = ms * 1e3
    k_us = k_ms * 1e3
    head_cfg = fsl.config_name(fsl.selected_config(B, D, V, packed=headline_packed))
    row_major = None
    if headline_packed:
        rfn, rkeep = make_step(B)
        r_ms = time_steps(torch, rfn, args.steps, args.warmup, stream)
        rk_ms, _, _, _ = measure_fused_kernel(torch, fsl, rfn, args.steps, args.warmup)
        row_major = {"config": fsl.config_name(fsl.selected_config(B, D, V)),
                     "us_per_step": round(r_ms * 1e3, 2), "launch_bracket_us": round(rk_ms * 1e3, 2),
                     "frac_of_roofline": round(roofline_us(B, D, V) / (r_ms * 1e3), 4)}
        del rkeep
    bytes_ = algorithmic_bytes(B, D, V)
    achieved_gbs = bytes_ / (k_us * 1e3)
    sweep = []
    for b in [int(x) for x in args.sweep.split(",") if x]:
        f, kp = make_step(b)
        t = time_steps(torch, f, args.sweep_steps, 10, stream) * 1e3
        q10, q50, q90 = step_percentiles(torch, f, args.sweep_steps, 5, stream)
        kt, _, _, _ = measure_fused_kernel(torch, fsl, f, args.sweep_steps, 5)
        kt *= 1e3
        entry = {"B": b, "config": fsl.config_name(fsl.selected_config(b, D, V)),
                 "us_per_step": round(t, 2),
                 "us_per_step_p10_p50_p90": [round(q10, 2), round(q50, 2), round(q90, 2)],
                 "launch_bracket_us": round(kt, 2),
                 "roofline_us": round(roofline_us(b, D, V), 2),
                 "frac_of_roofline": round(roofline_us(b, D, V) / t, 4),
                 "launch_hbm_GBs": round(algorithmic_bytes(b, D, V) / (kt * 1e3), 1),
                 "launch_mfma_TFLOPs": round(flops(b, D, V) / (kt * 1e6), 1),
                 "tokens_per_s": round(b / (t * 1e-6), 1)}
        if Wp is not None:
            pf, pkp = make_step(b, packed=True)
            pt = time_steps(torch, pf, args.sweep_steps, 10, stream) * 1e3
            r10, r50, r90 = step_percentiles(torch, pf, args.sweep_steps, 5, stream)
            pkt, _, _, _ = measure_fused_kernel(torch, fsl, pf, args.sweep_steps, 5)
            entry["packed_config"] = fsl.config_name(fsl.selected_config(b, D, V, packed=True))
            entry["packed_us_per_step"] = round(pt, 2)
            entry["packed_us_per_step_p10_p50_p90"] = [round(r10, 2), round(r50, 2), round(r90, 2)]
            entry["packed_launch_bracket_us"] = round(pkt * 1e3, 2)
            entry["packed_frac_of_roofline"] = round(roofline_us(b, D, V) / pt, 4)
            del pkp
        if not args.no_unfused:
            uf, ukp = make_step(b, unfused=True)
            ut = time_steps(torch, uf, max(10, args.sweep_steps // 4), 3, stream) * 1e3
            entry["unfused_us_per_step"] = round(ut, 2)
            entry["unfused_intermediate_bytes"] = 20 * b * V
            del ukp
        sweep.append(entry)
        del kp
    # Context, not a product path: the bf16 GEMM alone (B x V logits written to
    # HBM in bf16, no sampling) through torch.matmul, i.e. ROCm's BLAS library,
    # on the same row-major W.
    gemm_only = []
    for b in ((B, 256) if not args.no_gemm_context else ()):
        h_c = wl.make_h(wlk, b, dev)
        t = time_steps(torch, lambda i, h_c=h_c: torch.matmul(h_c, W.t()), 30, 5, stream) * 1e3
        gemm_only.append({"B": b, "us_per_call": round(t, 2),
                          "tflops": round(flops(b, D, V) / (t * 1e6), 1),
                          "fused_step_us": next((e.get("packed_us_per_step", e["us_per_step"])
                                                 for e in sweep if e["B"] == b), None)})
        del h_c
    torch.cuda.empty_cache()

    # Grouped (hierarchical) sampler: the vocabulary as G contiguous groups.
    # One step is fs_sample_groups_lse (every group's partials in one launch)
    # then fs_merge_lse; the same step as G fs_sample_partial_lse launches
    # (one per group) is timed beside it.
    grouped = []
    for b, G in ((B, 1), (B, 8), (256, 1), (256, 8)):
        if args.no_grouped or G < 1 or V % G:
            continue
        h_g = wl.make_h(wlk, b, dev)
        T_g = wl.make_temperature(wlk, b, dev)
        pv = torch.empty(G, b, dtype=torch.float32, device=dev)
        pi = torch.empty(G, b, dtype=torch.int32, device=dev)
        pl = torch.empty(G, b, dtype=torch.float32, device=dev)
        Vg = V // G
        cuts = [p * Vg for p in range(G + 1)]
        ws1 = fsl.alloc_workspace(fsl.groups_workspace_bytes(b, D, V, G), dev)
        wsg = fsl.alloc_workspace(fsl.workspace_bytes(b, D, Vg), dev)
        outs = (torch.empty(b, dtype=torch.int32, device=dev),
                torch.empty(b, dtype=torch.float32, device=dev),
                torch.empty(b, dtype=torch.float32, device=dev))
        W_g = Wp if Wp is not None else W

        def one(i, h_g=h_g, T_g=T_g, pv=pv, pi=pi, pl=pl, ws1=ws1, outs=outs, cuts=cuts):
            seed, step = wlk.sampler_seed(i)
            fsl.sample_groups_lse(h_g, W_g, T_g, seed, step, cuts, out=(pv, pi, pl),
                                  workspace=ws1, V=V)
            fsl.merge_lse(pv, pi, pl, T_g, seed, step, out=outs)

        def sep(i, h_g=h_g, T_g=T_g, pv=pv, pi=pi, pl=pl, wsg=wsg, outs=outs, G=G, Vg=Vg):
            seed, step = wlk.sampler_seed(i)
            for p in range(G):
                if Wp is not None:  # group p of the fragment-order W (Vg % 16 == 0)
                    fsl.sample_partial_lse(h_g, Wp[p * Vg * D:(p + 1) * Vg * D], T_g, seed, step,
                                           p * Vg, pv[p], pi[p], pl[p], workspace=wsg, V=Vg)
                else:
                    fsl.sample_partial_lse(h_g, W[p * Vg:(p + 1) * Vg], T_g, seed, step, p * Vg,
                                           pv[p], pi[p], pl[p], workspace=wsg)
            fsl.merge_lse(pv, pi, pl, T_g, seed, step, out=outs)
        # replayed as captured graphs so that host-side call overhead does not
        # stand in for device time
        times = {}
        for name, fn in (("one_launch", one), ("per_group_launches", sep)):
            for i in range(3):
                fn(i)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                fn(7)
            times[name] = time_steps(torch, lambda i: graph.replay(),
                                     max(10, args.sweep_steps // 2), 5,
                                     torch.cuda.current_stream(dev)) * 1e3
            torch.cuda.synchronize()
            del graph
        plain = next((e.get("packed_us_per_step" if Wp is not None else "us_per_step")
                      for e in sweep if e["B"] == b), None)
        cfg = fsl.selected_config(b, D, V, packed=Wp is not None, grouped=True)
        grouped.append({"B": b, "groups": G, "us_per_step": round(times["one_launch"], 2),
                        "per_group_launches_us_per_step": round(times["per_group_launches"], 2),
                        "config": fsl.config_name(cfg),
                        "w_layout": "fragment order" if Wp is not None else "row-major",
                        "whole_vocabulary_us_per_step": plain,
                        "ratio_to_whole_vocabulary": (round(times["one_launch"] / plain, 3)
                                                      if plain else None)})
        del h_g, T_g, pv, pi, pl, ws1, wsg, outs

    # Online sampler with early finalisation: fs_sample_online per step over
    # the vocabulary in 8 chunks of 16032 rows, or in 2 chunks (the first
    # 16032 rows, then the rest), replayed as a captured graph (1 + 2 chunks
    # launches).  "confident" weights (the first chunk holds a row aligned
    # with each hidden state, later rows are small) finalise every row after
    # the first chunk; the random weights never finalise early, which
    # measures the cost of chunking.  The bounds are computed once per weight
    # matrix and chunking (timed separately).
    online = []
    if not args.no_online:
        splits = (list(range(0, V + 1, V // 8)), [0, V // 8, V])
        for b in (B, 256):
            h_o = wl.make_h(wlk, b, dev)
            T_o = wl.make_temperature(wlk, b, dev)
            outs = (torch.empty(b, dtype=torch.int32, device=dev),
                    torch.empty(b, dtype=torch.float32, device=dev),
                    torch.empty(b, dtype=torch.int32, device=dev))
            for kind in ("confident", "random"):
                W_o = (wl.make_confident_w(wlk, h_o, chunk_rows=V // 8, later_std=0.002,
                                           device=dev) if kind == "confident" else W)
                # chunks run on the fragment-order copy when there is one
                W_run = (fsl.pack_weights(W_o) if kind == "confident" else Wp) if Wp is not None \
                    else W_o
                for cuts in splits:
                    n_chunks = len(cuts) - 1
                    bt = time_steps(torch, lambda i: fsl.online_bounds(W_o, cuts), 3, 1,
                                    stream) * 1e3
                    later = fsl.online_bounds(W_o, cuts)
                    ws = fsl.alloc_workspace(fsl.online_workspace_bytes(b, D, V, n_chunks), dev)

                    def ofn(i, h_o=h_o, T_o=T_o, W_run=W_run, cuts=cuts, later=later, outs=outs,
                            ws=ws):
                        seed, step = wlk.sampler_seed(i)
                        fsl.sample_online(h_o, W_run, T_o, seed, step, cuts, later, out=outs,
                                          workspace=ws, V=V)
                    for i in range(3):
                        ofn(i)
                    torch.cuda.synchronize()
                    graph = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(graph):
                        ofn(11)
                    ot = time_steps(torch, lambda i: graph.replay(),
                                    max(10, args.sweep_steps // 2), 5,
                                    torch.cuda.current_stream(dev)) * 1e3
                    torch.cuda.synchronize()
                    used = outs[2].float().mean().item()
                    del graph
                    plain = next((e.get("packed_us_per_step" if Wp is not None else "us_per_step")
                                  for e in sweep if e["B"] == b), None)
                    online.append({"B": b, "weights": kind, "chunks": n_chunks,
                                   "w_layout": "fragment order" if Wp is not None else "row-major",
                                   "first_chunk_rows": cuts[1],
                                   "us_per_step": round(ot, 2),
                                   "mean_chunks_used": round(used, 3),
                                   "whole_vocabulary_us_per_step": plain, "bounds_us": round(bt, 1)})
                    del later, ws
                del W_o, W_run
            del h_o, T_o, outs
            torch.cuda.empty_cache()

    # The other LM-head shapes (fused step only): Qwen3-shaped (D=5120,
    # V=151936, mixed temperatures with greedy rows), large batch (D=8192) and
    # one GPU's share of an 8-way vocabulary shard (D=8192, V=16032 at
    # vocab_offset 48096).  The shard's W (263 MB) would stay in the 256 MB
    # last-level cache between steps, so its steps rotate over four copies
    # (1.05 GB, "cold"); the same-copy rate is reported beside it ("hot").
    workloads = []
    if not args.no_workloads:
        del_keep = None
        for wk, Bs, copies in ((wl.QWEN3, (64, 128, 256), 1), (wl.LARGE_BATCH, (256, 512), 1),
                               (wl.TP8_SHARD, (1, 64, 256), 4)):
            Ws = [wl.make_w(wk, dev) for _ in range(copies)]
            Wps = [fsl.pack_weights(x, wk.vocab_offset) for x in Ws] if not args.no_packed else []
            for b in Bs:
                h_w = wl.make_h(wk, b, dev)
                T_w = wl.make_temperature(wk, b, dev)
                out_w = (torch.empty(b, dtype=torch.int32, device=dev),
                         torch.empty(b, dtype=torch.float32, device=dev))
                ws_w = fsl.alloc_workspace(fsl.workspace_bytes(b, wk.D, wk.V), dev)

                def wfn(i, Ws=Ws, h_w=h_w, T_w=T_w, out_w=out_w, ws_w=ws_w, wk=wk, rot=True):
                    seed, step = wk.sampler_seed(i)
                    fsl.sample(h_w, Ws[i % len(Ws) if rot else 0], T_w, seed, step,
                               vocab_offset=wk.vocab_offset, out=out_w, workspace=ws_w)
                t = time_steps(torch, wfn, max(20, args.sweep_steps // 2), 5, stream) * 1e3
                roof = max(2 * wk.V * wk.D / (HBM_PEAK_GBS * 1e3),
                           flops(b, wk.D, wk.V) / (MFMA_BF16_PEAK_TFLOPS * 1e6))
                e = {"workload": wk.name, "B": b, "D": wk.D, "V": wk.V,
                     "vocab_offset": wk.vocab_offset,
                     "config": fsl.config_name(fsl.selected_config(b, wk.D, wk.V)),
                     "us_per_step": round(t, 2), "roofline_us": round(roof, 2),
                     "frac_of_roofline": round(roof / t, 4)}
                if copies > 1:
                    th = time_steps(torch, lambda i: wfn(i, rot=False), max(20, args.sweep_steps // 2),
                                    5, stream) * 1e3
                    e["w_copies_rotated"] = copies
                    e["hot_us_per_step"] = round(th, 2)
                if Wps:
                    def pfn(i, Wps=Wps, h_w=h_w, T_w=T_w, out_w=out_w, ws_w=ws_w, wk=wk):
                        seed, step = wk.sampler_seed(i)
                        fsl.sample_packed(h_w, Wps[i % len(Wps)], wk.V, T_w, seed, step,
                                          vocab_offset=wk.vocab_offset, out=out_w, workspace=ws_w)
                    tp = time_steps(torch, pfn, max(20, args.sweep_steps // 2), 5, stream) * 1e3
                    e["packed_config"] = fsl.config_name(fsl.selected_config(b, wk.D, wk.V, packed=True))
                    e["packed_us_per_step"] = round(tp, 2)
                    e["packed_frac_of_roofline"] = round(roof / tp, 4)
                if wk is wl.LARGE_BATCH and b == 512 and not args.no_gemm_context:
                    tg = time_steps(torch, lambda i: torch.matmul(h_w, Ws[0].t()), 10, 3,
                                    stream) * 1e3
                    e["gemm_only_torch_matmul_us"] = round(tg, 2)
                    torch.cuda.empty_cache()
                workloads.append(e)
                del h_w, T_w, out_w, ws_w
            del Ws, Wps
            torch.cuda.empty_cache()

    unf_us = None
    if not args.no_unfused:
        uf, ukp = make_step(B, unfused=True)
        unf_us = time_steps(torch, uf, max(20, args.steps // 4), 5, stream) * 1e3
        del ukp

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        h_cpu = wl.bf16_bits(keep[0])
        T_cpu = keep[1].cpu().numpy()
        W_cpu = wl.bf16_bits(W)
        rows = list(range(B))
        times = []
        for i in range(3):  # median of three full steps
            t0 = time.perf_counter()
            oracle.sample(h_cpu, W_cpu, T_cpu, *wlk.sampler_seed(i), rows=rows)
            times.append(time.perf_counter() - t0)
        dt = sorted(times)[1]
        cores = oracle.max_threads()
        oracle.set_threads(1)  # and one single-threaded B=1 step
        t0 = time.perf_counter()
        oracle.sample(h_cpu[:1], W_cpu, T_cpu[:1], *wlk.sampler_seed(0))
        dt1 = time.perf_counter() - t0
        oracle.set_threads(0)
        # each workload's largest batch, timed on a sample of as many rows as
        # the oracle has threads (one row per thread: every row is an
        # independent full pass over the vocabulary) and scaled to the batch
        per_wl = []
        for wk, Bw in ((wl.TINY, 4), (wlk, 32), (wl.QWEN3, 256), (wl.LARGE_BATCH, 512),
                       (wl.TP8_SHARD, 256)):
            n_rows = min(Bw, cores)
            Wk = W_cpu if wk is wlk else wl.bf16_bits(wl.make_w(wk, "cpu" if wk.w_bytes() < (64 << 20)
                                                              else dev))
            hk = wl.bf16_bits(wl.make_h(wk, Bw, "cpu"))
            Tk = wl.make_temperature(wk, Bw, "cpu").numpy()
            t0 = time.perf_counter()
            oracle.sample(hk, Wk, Tk, *wk.sampler_seed(0), vocab_offset=wk.vocab_offset,
                          rows=list(range(n_rows)))
            dtk = time.perf_counter() - t0
            per_wl.append({"workload": wk.name, "B": Bw, "rows_timed": n_rows,
                           "s_per_step": round(dtk * -(-Bw // n_rows), 6)})
            del Wk
        cpu = {"value": round(dt * 1e6 * B / len(rows), 1), "unit": "µs/step",
               "cores": cores, "kind": "oracle", "cpu_model": cpu_model(),
               "sample": f"three full decode steps of the B={B} workload (all {len(rows)} rows, "
                         f"full V={V}, fp64 dot products), median {dt:.2f} s wall",
               "single_thread_b1_us_per_step": round(dt1 * 1e6, 1),
               "per_workload": per_wl}

    line = {
        "metric": METRIC, "value": round(us, 2), "unit": "µs/step", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02^2) weights, RMS-normalised N(0,1) hidden states)",
        "config": {"workload": wlk.name, "B": B, "D": D, "V": V, "temperature": 1.0,
                   "fresh_seed_per_step": True,
                   "w_layout": ("fragment order, packed once at load (fs_pack_weights)"
                                if headline_packed else "row-major [V][D]")},
        "tokens_per_s": round(B / (us * 1e-6), 1),
        "frac_of_roofline": round(roofline_us(B, D, V) / us, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(B, head_cfg),
                     "kernel": head_cfg,
                     "kernel_sources_sha256": kernel_sources_sha256()[:16],
                     "launch_bracket_avg_us": round(k_us, 2),
                     "launch_bracket_min_us": round(k_lo * 1e3, 2),
                     "launch_bracket_max_us": round(k_hi * 1e3, 2), "launches": k_n,
                     "duration_source": "HIP events on the launch stream around each fused-kernel "
                                        "launch (kernel plus its dispatch; the tile merge is outside)",
                     "algorithmic_bytes_per_launch": bytes_},
        "us_per_step_p10_p50_p90": [round(p10, 2), round(p50, 2), round(p90, 2)],
        "row_major": row_major,
        "unfused_us_per_step": round(unf_us, 2) if unf_us is not None else None,
        "cpu_baseline": cpu,
        "sweep": sweep,
        "grouped_lse": grouped,
        "gemm_only_torch_matmul": gemm_only,
        "online": online,
        "other_workloads": workloads,
        "device": {"name": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
                   **device_peaks(fsl, dev)},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
