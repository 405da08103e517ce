"""Benchmark of the linear-attention state-caching hot path on one MI355X.

Step (the headline): a cold 32768-token prompt of 8 segments x 4096 tokens,
gated delta rule with 32 value heads over 16 key heads, d = 128, bf16 inputs:
build the cached pair (T_C, S_{C|0}) of every (segment, head), then compose
the 8 pairs into the prompt's end state.  value = prompt tokens per second.

Second leg (reported under "compose"): a ~100k-token prompt of 100 segments x
1024 tokens, 32 heads, d = 128, composed from pre-built fp32 pairs with a
w = 8 seam window (width-4 causal conv warm-up) at each of the 99 inner
segments.  value = segment compositions per second.

Inputs are synthetic (seeded), resident in HBM before timing starts.  The
per-kernel averages behind the roofline figures come from HIP events on the
stream the kernels run on.  ``cpu_baseline`` times the fp64 CPU oracle on a
bounded sample of the headline workload.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--leg build|compose|all]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "segment-build tokens/s + compositions/s per GPU, % of MFMA/HBM roofline"
PEAK_MFMA_F16 = 2500.0     # TFLOP/s, MI355X dense fp16/bf16 matrix cores
PEAK_HBM = 8000.0          # GB/s, MI355X HBM3E
PEAK_MFMA_F32 = 157.3      # TFLOP/s, MI355X dense fp32 matrix cores

# HBM traffic per launch comes from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
# summarised in profiles/hbm_counters.md; a row counts only while the digest of
# the kernel's sources still matches the one recorded with the counters.
CSRC = os.path.join(ROOT, "state_caching_amd", "csrc")
KERNEL_SOURCES = {
    "build_delta_f16_kernel": ["build_delta_f16.hip", "common.h", "launch.h"],
    "seam_ops_kernel": ["seam.h", "compose_split.hip", "common.h", "launch.h"],
    "compose_split_kernel": ["compose_split.hip", "seam.h", "common.h", "launch.h"],
    "compose_group_kernel": ["compose_group.hip", "seam.h", "common.h", "launch.h"],
    "build_kda_kernel": ["build_kda.hip", "common.h", "launch.h"],
    "rope_keys_kernel": ["rope.hip", "common.h", "launch.h"],
    "seam_readout_kernel": ["compose_split.hip", "seam.h", "common.h", "launch.h"],
}


def source_digest(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:12]


def counter_traffic(kernels, workload_tag):
    """Scaled HBM bytes per launch summed over `kernels`, or None when any row
    is missing or was taken on sources that have changed since."""
    path = os.path.join(ROOT, "profiles", "hbm_counters.md")
    if not os.path.exists(path):
        return None
    rows = {}
    fetch_scale = write_scale = None
    with open(path) as f:
        for line in f:
            m = re.match(r"^fetch_scale:\s*([0-9.]+)\s*$", line)
            if m: fetch_scale = float(m.group(1))
            m = re.match(r"^write_scale:\s*([0-9.]+)\s*$", line)
            if m: write_scale = float(m.group(1))
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) == 6 and cells[0] in KERNEL_SOURCES:
                try:
                    rows[(cells[0], cells[1])] = (cells[2], float(cells[3]), float(cells[4]))
                except ValueError:
                    pass
    if fetch_scale is None or write_scale is None:
        return None
    total = 0.0
    for k in kernels:
        r = rows.get((k, workload_tag))
        if r is None or r[0] != source_digest(k):
            return None
        total += (r[1] * fetch_scale + r[2] * write_scale) * 1024.0
    return total


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_flops(n_tokens, h_v, d_k, d_v):
    # algorithmic work of the gated-delta build: 4 d_k (d_k + d_v) flop per token per value head
    return 4.0 * d_k * (d_k + d_v) * n_tokens * h_v


def build_bytes(wl):
    import torch
    el = 2 if wl.dtype == torch.bfloat16 else 4
    n = wl.n_tokens
    inputs = n * (wl.h_k * wl.d_k + wl.h_v * wl.d_v + 2 * wl.h_v) * el
    outputs = wl.n_seg * wl.h_v * (wl.d_k * wl.d_k + wl.d_k * wl.d_v) * 4
    return inputs + outputs


def compose_bytes(wl):
    """Algorithmic bytes of a dense compose with seams: every pair read once,
    each seam window's raw rows, tails and gates read once, conv weights once,
    the state written once."""
    el = 2
    n, H, d = wl.n_seg, wl.h_v, wl.d_k
    pairs = n * H * (d * d + d * d) * 4
    n_win = n - 1
    W = wl.conv_w
    seam = n_win * (wl.seam_w * (wl.h_k * d + H * d + 2 * H) + (W - 1) * (wl.h_k * d + H * d)) * el
    weights = (wl.h_k * d + H * d) * W * 4
    return pairs + seam + weights + H * d * d * 4


def compose_flops(wl):
    n, H, d = wl.n_seg, wl.h_v, wl.d_k
    return 2.0 * d * d * d * n * H


def time_leg(fn, steps, warmup, torch, events):
    """Run fn() warmup + steps times; returns (wall ms per step, per-kernel ms lists)."""
    for _ in range(warmup):
        fn(None)
    torch.cuda.synchronize()
    per = {k: [] for k in events}
    recs = []
    t0 = time.perf_counter()
    for _ in range(steps):
        ev = {k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for k in events}
        fn(ev)
        recs.append(ev)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    for ev in recs:
        for k, (a, b) in ev.items():
            per[k].append(a.elapsed_time(b))
    return wall, per


def cpu_baseline(wl, target_s=12.0):
    """The fp64 oracle on a bounded sample of (segment, head) build units."""
    import numpy as np
    import oracle
    oracle.build()
    thr = oracle.threads()
    units = [(s, h) for s in range(wl.n_seg) for h in range(wl.h_v)]
    # one unit first to size the sample
    t0 = time.perf_counter()
    oracle.build_pairs(wl, segs=[0], heads=[0])
    t1 = time.perf_counter() - t0
    n = int(max(thr, min(len(units), thr * max(1, round(target_s / max(t1, 1e-3))))))
    n = max(1, min(n, len(units)))
    rng = np.random.default_rng(0)
    pick = [units[i] for i in sorted(rng.choice(len(units), n, replace=False))]
    by_seg = {}
    for s, h in pick:
        by_seg.setdefault(s, []).append(h)
    t0 = time.perf_counter()
    for s, hs in by_seg.items():
        oracle.build_pairs(wl, segs=[s], heads=hs)
    dt = time.perf_counter() - t0
    frac = n / len(units)
    tok_s = frac * wl.n_tokens / dt
    return {"value": tok_s, "unit": "tokens/s", "cores": thr, "kind": "oracle",
            "sample": f"{n} of {len(units)} (segment, value-head) pair builds of the headline "
                      f"workload (4096 tokens each, fp64 token-by-token, two runs per pair), "
                      f"{dt:.1f} s wall on {thr} threads; tokens/s scaled by {n}/{len(units)}"}


def measured_peaks(torch, dev):
    """What this GPU reaches on plain library work, beside the published peaks
    the roofline fractions use: a 1 GiB device-to-device copy (read + write
    bytes) and a bf16 8192^3 GEMM (torch.matmul)."""
    log("measuring a device copy and a bf16 GEMM for context")
    x = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    x.fill_(1.0)
    for _ in range(2):
        y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * x.numel() * 4 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del x, y
    n = 8192
    a = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    b = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    for _ in range(2):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    gemm_tf = 2.0 * n ** 3 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b
    torch.cuda.empty_cache()
    return {"hbm_copy_GBps": copy_gbs, "bf16_gemm_TFLOPs": gemm_tf,
            "note": "context only; roofline fractions use the published peaks"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--leg", choices=["build", "compose", "kda", "rope", "all"], default="all")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import torch
    import synth
    from state_caching_amd.runner import DeviceWorkload

    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda:0")
    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16-in/fp16-mfma/fp32-acc", "data": "synthetic"}

    if args.calib_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if args.leg in ("build", "all"):
        log("generating the 32k-token cold prompt (8 x 4096, 32/16 heads, d=128, bf16)")
        wl3 = synth.workload("gdn_gqa_d128_8x4096_bf16")
        dw3 = DeviceWorkload(wl3, dev)
        T = torch.empty((wl3.n_seg, wl3.h_v, 128, 128), dtype=torch.float32, device=dev)
        S0 = torch.empty_like(T)
        S = torch.empty((wl3.h_v, 128, 128), dtype=torch.float32, device=dev)
        from state_caching_amd import segment_build, compose

        def step(ev):
            if ev: ev["build"][0].record()
            segment_build(dw3.rule, dw3.gate_kind, dw3.k, dw3.v, dw3.beta, dw3.gate,
                          dw3.seg_start, dw3.seg_len, T_out=T, S0_out=S0)
            if ev: ev["build"][1].record(); ev["compose"][0].record()
            compose(T, S0, list(range(wl3.n_seg)), tform=dw3.tform, prec=dw3.prec, S_out=S)
            if ev: ev["compose"][1].record()

        log(f"timing {args.steps} steps (+{args.warmup} warm-up)")
        wall, per = time_leg(step, args.steps, args.warmup, torch, ["build", "compose"])
        kb = sum(per["build"]) / len(per["build"])
        kc = sum(per["compose"]) / len(per["compose"])
        fl = build_flops(wl3.n_tokens, wl3.h_v, wl3.d_k, wl3.d_v)
        ach = fl / (kb * 1e-3) / 1e12
        out.update({
            "value": wl3.n_tokens / (wall * 1e-3), "unit": "tokens/s",
            "ms_per_step": wall,
            "config": {"workload": "cold prompt, gated delta (GDN), 32768 tokens = 8 segments x 4096, "
                                   "32 value heads over 16 key heads (GQA), d_k = d_v = 128, bf16 "
                                   "inputs, fp32 pairs: build all (segment, head) pairs then compose",
                       "segments": wl3.n_seg, "seg_len": 4096, "h_v": wl3.h_v, "h_k": wl3.h_k,
                       "d": 128, "in_dtype": "bf16"},
            "roofline": {"bound": "mfma", "kernel": "build_delta_f16_kernel<128,bf16,bf16,bf16>",
                         "achieved": ach, "peak": PEAK_MFMA_F16, "unit": "TFLOP/s",
                         "frac": ach / PEAK_MFMA_F16,
                         "traffic": counter_traffic(["build_delta_f16_kernel"], "gdn_32k_prompt"),
                         "kernel_ms": kb, "algorithmic_flop": fl,
                         "algorithmic_bytes": build_bytes(wl3)},
            "build_tokens_per_s": wl3.n_tokens / (kb * 1e-3),
            "build_pairs_per_s": wl3.n_seg * wl3.h_v / (kb * 1e-3),
            "compose_cold_ms": kc,
        })
        del dw3, T, S0, S
        torch.cuda.empty_cache()

    if args.leg in ("compose", "all"):
        log("generating the 100 x 1024-token prompt with conv and seams (32 heads, d=128, bf16)")
        wl4 = synth.workload("gdn_d128_32h_100x1024_seams_bf16")
        dw4 = DeviceWorkload(wl4, dev)
        T4, S04 = dw4.build()          # pre-built pairs (not timed)
        S4 = torch.empty((wl4.h_v, 128, 128), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        from state_caching_amd import compose

        order = list(range(wl4.n_seg))

        def step4(ev):
            if ev: ev["compose"][0].record()
            compose(T4, S04, order, tform=dw4.tform, prec=dw4.prec, seams=dw4.seams, S_out=S4)
            if ev: ev["compose"][1].record()

        wall4, per4 = time_leg(step4, args.steps, args.warmup, torch, ["compose"])
        k4 = sum(per4["compose"]) / len(per4["compose"])
        by = compose_bytes(wl4)
        gbs = by / (k4 * 1e-3) / 1e9
        comp = {"workload": "hot prompt, gated delta, 100 segments x 1024 tokens, 32 heads, d = 128, "
                            "pre-built fp32 pairs, w = 8 seam window with width-4 conv at 99 inner segments",
                "compositions_per_s": wl4.n_seg / (k4 * 1e-3),
                "head_compositions_per_s": wl4.n_seg * wl4.h_v / (k4 * 1e-3),
                "ms_per_compose": k4, "wall_ms_per_step": wall4,
                "roofline": {"bound": "hbm",
                             "kernel": "hypic_compose = seam_ops_kernel<128> + compose_group_kernel<128,seams> "
                                       "(groups of 13 positions) + compose_split_kernel<128> (8 group pairs)",
                             "achieved": gbs, "peak": PEAK_HBM, "unit": "GB/s",
                             "frac": gbs / PEAK_HBM,
                             "traffic": counter_traffic(["seam_ops_kernel", "compose_group_kernel", "compose_split_kernel"],
                                                        "gdn_100_segments_seams"),
                             "algorithmic_bytes": by,
                             "mfma_tflops": compose_flops(wl4) / (k4 * 1e-3) / 1e12}}
        # the same compose with the read-outs of all 99 windows (queries of every
        # window token in, o_t = q_t^T S_t out)
        import copy
        import numpy as np
        n_win, w4 = len(wl4.window_ranges()), wl4.seam_w
        rng = np.random.default_rng(4004)
        q4 = synth._round(rng.standard_normal((n_win, w4, wl4.h_k, wl4.d_k)) / np.sqrt(wl4.d_k),
                          wl4.dtype).to(dev)
        sm_ro = copy.copy(dw4.seams)
        sm_ro.q = q4
        sm_ro.o = torch.empty((n_win, w4, wl4.h_v, wl4.d_v), dtype=torch.float32, device=dev)

        def step4r(ev):
            if ev: ev["compose"][0].record()
            compose(T4, S04, order, tform=dw4.tform, prec=dw4.prec, seams=sm_ro, S_out=S4)
            if ev: ev["compose"][1].record()

        _, per4r = time_leg(step4r, args.steps, args.warmup, torch, ["compose"])
        k4r = sum(per4r["compose"]) / len(per4r["compose"])
        by_r = by + q4.numel() * q4.element_size() + sm_ro.o.numel() * 4
        gbs_r = by_r / (k4r * 1e-3) / 1e9
        comp["readouts"] = {"workload": "the same compose with the read-outs of all 99 windows (8 tokens each, "
                                        "bf16 queries of 16 key heads in, fp32 outputs of 32 heads out)",
                            "ms_per_compose": k4r, "overhead_ms": k4r - k4,
                            "roofline": {"bound": "hbm",
                                         "kernel": "hypic_compose with read-outs: seam_ops_kernel + compose_group_kernel"
                                                   "<128,seams,read-outs> + compose_split_kernel (group-start states) "
                                                   "+ seam_readout_kernel<128>",
                                         "achieved": gbs_r, "peak": PEAK_HBM, "unit": "GB/s",
                                         "frac": gbs_r / PEAK_HBM,
                                         "traffic": counter_traffic(["seam_ops_kernel", "compose_group_kernel",
                                                                     "compose_split_kernel", "seam_readout_kernel"],
                                                                    "gdn_100_segments_readouts"),
                                         "algorithmic_bytes": by_r}}
        del sm_ro, q4
        out["compose"] = comp
        if "value" not in out:
            out.update({"value": comp["compositions_per_s"], "unit": "compositions/s",
                        "ms_per_step": wall4,
                        "config": {"workload": comp["workload"]}, "roofline": comp["roofline"]})

    if args.leg in ("kda", "all"):
        log("generating the 32k-token prompt with diagonal gates (KDA; 8 x 4096, 32/16 heads, d=128, bf16)")
        wl5 = synth.workload("kda_gqa_d128_8x4096_bf16")
        dw5 = DeviceWorkload(wl5, dev)
        T5 = torch.empty((wl5.n_seg, wl5.h_v, 128, 128), dtype=torch.float32, device=dev)
        S05 = torch.empty_like(T5)
        from state_caching_amd import segment_build

        def step5(ev):
            if ev: ev["kda"][0].record()
            segment_build(dw5.rule, dw5.gate_kind, dw5.k, dw5.v, dw5.beta, dw5.gate,
                          dw5.seg_start, dw5.seg_len, T_out=T5, S0_out=S05)
            if ev: ev["kda"][1].record()

        wall5, per5 = time_leg(step5, args.steps, args.warmup, torch, ["kda"])
        k5 = sum(per5["kda"]) / len(per5["kda"])
        # per token and value head: the gate on [T | S], k^T of it and the rank-one
        # update, 5 d_k (d_k + d_v) flop
        fl5 = 5.0 * wl5.n_tokens * wl5.h_v * wl5.d_k * (wl5.d_k + wl5.d_v)
        ach5 = fl5 / (k5 * 1e-3) / 1e12
        out["kda"] = {"workload": "cold prompt, delta rule with a diagonal gate (KDA), 32768 tokens = "
                                  "8 segments x 4096, 32 value heads over 16 key heads, d = 128, bf16 "
                                  "inputs, fp32 pairs",
                      "ms_per_build": k5, "tokens_per_s": wl5.n_tokens / (k5 * 1e-3),
                      "roofline": {"bound": "mfma", "kernel": "build_kda_kernel<128,bf16,bf16> (fp32 products)",
                                   "achieved": ach5, "peak": PEAK_MFMA_F32, "unit": "TFLOP/s",
                                   "frac": ach5 / PEAK_MFMA_F32,
                                   "traffic": counter_traffic(["build_kda_kernel"], "kda_32k_prompt"),
                                   "algorithmic_flop": fl5}}
        del dw5, T5, S05
        torch.cuda.empty_cache()

    if args.leg in ("rope", "all"):
        log("rotary re-rotation of the cached keys of a 32k-token prompt (16 heads, d=128, bf16)")
        from state_caching_amd import rope_rerotate
        r6 = synth.ROPE_32K
        n6, h6 = r6["n_tokens"], r6["h"]
        K6 = synth.rope_keys(r6["seed"], n6, h6, r6["d"]).to(dev)
        K6o = torch.empty_like(K6)
        st6, ln6, dl6 = r6["seg_start"], r6["seg_len"], r6["delta"]

        def step6(ev):
            if ev: ev["rope"][0].record()
            rope_rerotate(K6, st6, ln6, dl6, out=K6o)
            if ev: ev["rope"][1].record()

        wall6, per6 = time_leg(step6, args.steps, args.warmup, torch, ["rope"])
        k6 = sum(per6["rope"]) / len(per6["rope"])
        by6 = 2.0 * K6.numel() * K6.element_size()     # every key read once and written once
        gbs6 = by6 / (k6 * 1e-3) / 1e9
        out["rope"] = {"workload": "cached full-attention keys of a 32768-token prompt (8 segments x 4096, "
                                   "16 KV heads, d = 128, bf16) moved to new start positions, out of place",
                       "ms_per_call": k6, "rows_per_s": n6 * h6 / (k6 * 1e-3),
                       "roofline": {"bound": "hbm", "kernel": "rope_keys_kernel<bf16, half pairs>",
                                    "achieved": gbs6, "peak": PEAK_HBM, "unit": "GB/s", "frac": gbs6 / PEAK_HBM,
                                    "traffic": counter_traffic(["rope_keys_kernel"], "rope_32k_keys"),
                                    "algorithmic_bytes": by6}}
        del K6, K6o
        torch.cuda.empty_cache()

    if args.leg == "all":
        out["measured_peaks"] = measured_peaks(torch, dev)
    if not args.no_cpu:
        log("timing the fp64 oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(synth.workload("gdn_gqa_d128_8x4096_bf16"))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
