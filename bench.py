"""Benchmark: one decode step of the paged MLA hot path on one MI355X.

A step is the whole path on one batch: the split plan and the query
absorption (one launch, mla_absorb_q_with_plan; --separate-plan runs
mla_get_metadata and mla_absorb_q instead), mla_decode_paged (split kernel +
combine) and mla_up_v. The cache append
(mla_append_kv) is timed on its own after the steps and reported beside them. Inputs are seeded
synthetic tensors already resident in HBM. To keep the 256 MB Infinity Cache
from serving repeats, R copies of every input and output rotate, with R times
the working set above 1 GiB.

`value` is the wall time per step over exactly --steps steps replayed from HIP
graphs recorded through torch's graph capture on the library's stream: one graph
holds one step on each rotating input set (the graph launch cost spread over
those steps, as over the layers of a model in one graph), single-step graphs
cover the remainder, and no host launch gap sits between the kernels of a step. Before the timed steps, untimed steps run for
--warmup-seconds (the clock settles only under sustained load; reported as
`warmup_s`) and then --warmup steps; the graph replays get the same time-based
warm-up after capture (`graph_warmup_replays`), since the GPU idles while the
graphs are recorded. `eager_us_per_step` is at least 50 of the
same steps launched eagerly; hipEvents around each call give the medians in
`stage_us` and the decode call's `decode_us` and roofline. With the default
workload (full_heads) the matrix-bound multi_token workload is measured in the
same run and reported under its own key.

Prints one JSON line (rank 0, N = 1). Usage:
    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config full_heads]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode µs/call + latent-KV TB/s + TFLOPS (% roofline), b=128 h=128"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix peak


# bytes a cached token occupies: a bf16 row of 576 values, or a quantised row (512 e4m3 codes,
# 64 bf16 key values and its fp32 scale)
TOKEN_BYTES = {"bf16": 1152, "fp8": 512 + 128 + 4}


def algorithmic_work(inp, kv="bf16"):
    """Bytes and flops the decode call must move and compute (no re-reads, no partials)."""
    import numpy as np
    L = np.maximum(inp.seqlens.astype(np.int64), 0)
    rows = inp.b * inp.s_q * inp.h
    pages = (L + 63) // 64
    kv_bytes = int(L.sum()) * TOKEN_BYTES[kv]
    q_bytes = rows * (512 + 64) * 2
    out_bytes = rows * (512 * 2 + 4)
    int_bytes = 4 * int(pages.sum()) + 4 * inp.b
    keys = 0
    for j in range(inp.s_q):
        n = L - inp.s_q + 1 + j if inp.causal else L
        keys += int(np.maximum(n, 0).sum())
    flops = 2 * inp.h * keys * (576 + 512)
    return dict(kv_bytes=kv_bytes, bytes=kv_bytes + q_bytes + out_bytes + int_bytes, flops=flops)


def roofline_bound(work) -> str:
    """The roofline that bounds the decode call: the bf16 matrix peak when its algorithmic flops per
    algorithmic byte exceed the chip's balance point (2.5 PF/s over 8 TB/s, about 312 flop/B), else HBM."""
    ridge = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
    return "mfma" if work["flops"] / work["bytes"] > ridge else "hbm"


def roofline_entry(work, t_dec: float, traffic):
    """roofline object of the JSON line for a decode call of t_dec seconds."""
    bound = roofline_bound(work)
    if bound == "mfma":
        achieved, peak, unit = work["flops"] / t_dec / 1e12, MFMA_BF16_PEAK_TFS, "TFLOP/s"
    else:
        achieved, peak, unit = work["bytes"] / t_dec / 1e9, HBM_PEAK_GBS, "GB/s"
    return {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic,
            "traffic_unit": "HBM bytes per call (calibrated counters)",
            "kernel": "mla_decode_paged call (split kernel + combine)",
            "algorithmic_bytes": work["bytes"], "algorithmic_flops": work["flops"]}


TRAFFIC_SOURCES = ("mla_decode.hip", "mla_device.h", "mla_metadata.hip", "mla_plan.h")


def recorded_traffic(config: str):
    """HBM bytes per decode call from the calibrated FETCH_SIZE/WRITE_SIZE runs recorded under
    profiles/, or None when there is no record for this workload or the kernel sources changed since."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "mla_decode_paged_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    path = os.path.join(ROOT, "profiles", f"mla_decode_{config}.md")
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as f:
        m = re.search(r"^traffic-record: workload=(\S+) bytes_per_call=(\d+) sources_sha256=([0-9a-f]{64})$",
                      f.read(), re.M)
    if not m or m.group(1) != config or m.group(3) != h.hexdigest():
        return None
    return int(m.group(2))


def time_append(mla, inp, sets, n: int, kv: str = "bf16"):
    """The step's cache append (mla_append_kv) on the same workload, after the timed steps:
    hipEvent time per call over back-to-back calls and its HBM rate (new rows read and written
    once, plus ints)."""
    import numpy as np
    import torch

    from mla_inputs import make_new_rows
    new = torch.from_numpy(make_new_rows(inp, seed=1).view(np.int16)).view(torch.bfloat16).cuda()
    append = mla.append_kv_fp8 if kv == "fp8" else mla.append_kv  # the quantised cache quantises on append
    for s in sets[:2]:
        append(new, s["kv"], s["bt"], s["sl"])
    torch.cuda.synchronize()
    # The kernel is far shorter than one host-side launch, so the calls are queued behind a
    # sleeping kernel first: the events then see back-to-back launches, not host latency.
    torch.cuda._sleep(10_000_000)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        s = sets[i % len(sets)]
        append(new, s["kv"], s["bt"], s["sl"])
    e1.record()
    torch.cuda.synchronize()
    assert mla.take_device_error() == 0
    us = e0.elapsed_time(e1) * 1e3 / n
    nbytes = inp.b * inp.s_q * (1152 + TOKEN_BYTES[kv]) + 4 * inp.b * (1 + inp.s_q)
    return {"us": round(us, 3), "bytes": nbytes, "GBps": round(nbytes / us / 1e3, 1),
            "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 5)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, budget_s: float):
    """Time the CPU oracle as it stands (NumPy fp32, naive expand-then-attend form) on a bounded sample
    of the workload, with as many BLAS threads as this process may run on, and scale to one call."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import mla_oracle as O
    cores = len(os.sched_getaffinity(0))
    order = np.argsort(inp.seqlens)
    seqs = [int(order[len(order) // 2])]  # a median-length sequence
    done_heads = 0
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        for hd in range(inp.h):  # one head at a time until the budget is spent
            O.decode_naive_inputs(inp, seqs=seqs, heads=[hd], dtype=np.float32)
            done_heads += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
    L = np.maximum(inp.seqlens.astype(np.int64), 0)
    frac = float(L[seqs].sum()) * done_heads / (float(L.sum()) * inp.h)
    return {"value": round(dt / frac * 1e6, 1), "unit": "us/call", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "sampled_fraction": round(frac, 6), "sample_s": round(dt, 2),
            "sample": f"naive fp32 NumPy oracle on sequence {seqs[0]} (L={int(L[seqs[0]])}), {done_heads} of "
                      f"{inp.h} heads ({frac:.4%} of the call's key-head pairs), {dt:.1f} s with {cores} BLAS "
                      f"threads, scaled by key-head count to the full call"}


def _dev_bf16(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _dev_i32(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def measure(mla, inp, args, steps: int, warmup: int, warmup_s: float, kv: str = "bf16"):
    """One workload: R rotating input sets resident in HBM; a time-based warm-up (the clock settles only
    after about 100 steps of load), then ``warmup`` untimed steps; max(steps, 50) eager steps with
    hipEvents around every call (their medians give the per-call times); then the same steps captured
    in a HIP graph of R steps (one per input set) and in single-step graphs, replayed untimed for
    ``warmup_s`` seconds (the clock falls while the graphs are recorded) and ``warmup`` more steps,
    then exactly ``steps`` timed steps (the step time)."""
    import numpy as np
    import torch

    kv0 = _dev_bf16(inp.kv_cache)
    if kv == "fp8":  # the quantised cache, converted on the GPU
        kv0 = mla.quantize_pages(kv0)
        torch.cuda.synchronize()
    working = kv0.numel() * kv0.element_size() + inp.b * inp.s_q * inp.h * (576 + 512 + 512) * 2
    R = max(1, math.ceil((1 << 30) / working))
    decode = mla.decode_paged_fp8 if kv == "fp8" else mla.decode_paged
    sets = []
    for r in range(R):
        sets.append(dict(
            kv=kv0 if r == 0 else kv0.clone(), bt=_dev_i32(inp.block_table), sl=_dev_i32(inp.seqlens),
            q_nope=_dev_bf16(inp.q_nope), q_pe=_dev_bf16(inp.q_pe), w_uk=_dev_bf16(inp.w_uk),
            w_uv=_dev_bf16(inp.w_uv),
            q_lat=torch.empty((inp.b, inp.s_q, inp.h, 512), dtype=torch.bfloat16, device="cuda"),
            q_lo=torch.empty((inp.b, inp.s_q, inp.h, 512), dtype=torch.bfloat16, device="cuda"),
            o_lat=torch.empty((inp.b, inp.s_q, inp.h, 512), dtype=torch.bfloat16, device="cuda"),
            lse=torch.empty((inp.b, inp.s_q, inp.h), dtype=torch.float32, device="cuda"),
            o=torch.empty((inp.b, inp.s_q, inp.h, 128), dtype=torch.bfloat16, device="cuda")))
    slots = mla.num_slots(inp.b, inp.s_q, inp.h)
    for s in sets:
        s["meta"] = torch.empty((slots, mla.META_WORDS), dtype=torch.int32, device="cuda")
        s["ns"] = torch.empty((inp.b + 1,), dtype=torch.int32, device="cuda")
    ws = torch.empty((mla.workspace_bytes(inp.b, inp.s_q, inp.h, slots),), dtype=torch.uint8, device="cuda")

    first = ("meta", "absorb") if args.separate_plan else ("plan_absorb",)
    ev = {k: [] for k in first + ("decode", "up_v")}

    def step(i, timed):
        s = sets[i % R]
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if timed else None
        if timed:
            e[0].record()
        if args.separate_plan:
            meta, ns = mla.get_metadata(s["sl"], slots, s_q=inp.s_q, h=inp.h, out=(s["meta"], s["ns"]))
            if timed:
                e[1].record()
            mla.absorb_q(s["q_nope"], s["w_uk"], out=(s["q_lat"], s["q_lo"]))
        else:
            _, (meta, ns) = mla.absorb_q_with_plan(s["q_nope"], s["w_uk"], s["sl"],
                                                   out=((s["q_lat"], s["q_lo"]), (s["meta"], s["ns"])))
            if timed:
                e[1].record()
        if timed:
            e[2].record()
        decode(s["q_lat"], s["q_pe"], s["kv"], s["bt"], s["sl"], meta, ns, inp.scale, inp.causal,
               q_lat_lo=s["q_lo"], workspace=ws, out=(s["o_lat"], s["lse"]))
        if timed:
            e[3].record()
        mla.up_v(s["o_lat"], s["w_uv"], out=s["o"])
        if timed:
            e[4].record()
            stages = ((("meta", 0, 1), ("absorb", 1, 2)) if args.separate_plan else (("plan_absorb", 0, 1),))
            for k, a, b in stages + (("decode", 2, 3), ("up_v", 3, 4)):
                ev[k].append((e[a], e[b]))

    # time-based warm-up, then the requested warm-up steps
    t0 = time.perf_counter()
    n_time_warm = 0
    while time.perf_counter() - t0 < warmup_s:
        for _ in range(25):
            step(n_time_warm, False)
            n_time_warm += 1
        torch.cuda.synchronize()
    t_warm = time.perf_counter() - t0
    for i in range(warmup):
        step(i, False)
    torch.cuda.synchronize()
    n_ev = max(steps, 50)
    t0 = time.perf_counter()
    for i in range(n_ev):
        step(i, True)
    torch.cuda.synchronize()
    us_step_eager = (time.perf_counter() - t0) / n_ev * 1e6
    assert mla.take_device_error() == 0
    per_call = {k: [a.elapsed_time(b) * 1e3 for a, b in v] for k, v in ev.items()}
    # The same steps replayed from HIP graphs: each step's launches are
    # recorded once, so a replay has no host launch gaps between its kernels.
    us_step_graph = None
    n_graph_warm = 0
    if not args.no_graph:
        # One graph holds one step on each of the R rotating input sets, so the
        # launch cost of a graph is spread over R steps, as it is over the
        # layers of a model captured in one graph; single-step graphs cover a
        # step count that is not a multiple of R. Each step is the whole path
        # on its own batch: nothing is shared or skipped between them.
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all):
            for r in range(R):
                step(r, False)
        singles = []
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(r, False)
            singles.append(g)

        def replay(n):  # exactly n steps
            for _ in range(n // R):
                g_all.replay()
            for r in range(n % R):
                singles[r].replay()

        # The GPU idles while the graphs are recorded and its clock drops: the
        # first ~100 replays after capture run about 15 % slower. The replays
        # get the same time-based warm-up as the eager steps, then the
        # requested warm-up steps, before exactly `steps` timed steps.
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < warmup_s:
            replay(25 * R)
            n_graph_warm += 25 * R
            torch.cuda.synchronize()
        replay(max(warmup, R))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        replay(steps)
        torch.cuda.synchronize()
        us_step_graph = (time.perf_counter() - t0) / steps * 1e6
        assert mla.take_device_error() == 0
        del g_all, singles
    out = dict(sets=sets, R=R, slots=slots, us_step_eager=us_step_eager, us_step_graph=us_step_graph,
               n_ev=n_ev, t_warm=t_warm, n_time_warm=n_time_warm, n_graph_warm=n_graph_warm,
               median={k: float(np.median(v)) for k, v in per_call.items()},
               mean={k: float(np.mean(v)) for k, v in per_call.items()})
    return out


def summary(inp, m, traffic, seed, kv="bf16"):
    """Per-workload figures of the JSON line for one measure() result."""
    work = algorithmic_work(inp, kv)
    t_dec = m["median"]["decode"] * 1e-6
    achieved = work["bytes"] / t_dec / 1e9
    tflops = work["flops"] / t_dec / 1e12
    from mla_inputs import CONFIGS
    cfg = CONFIGS[inp.name]
    us_step = m["us_step_graph"] if m["us_step_graph"] is not None else m["us_step_eager"]
    lens = cfg["seqlens"]
    if len(set(inp.seqlens.tolist())) == 1 and lens != ("all", int(inp.seqlens[0])):  # a --seqlen point
        lens = ("all", int(inp.seqlens[0]))
    cache = "bf16 576-wide rows" if kv == "bf16" else "quantised rows (e4m3 latent + bf16 key + fp32 scale, 644 B)"
    return {
        "workload": f"{inp.name}: b={inp.b} h={inp.h} s_q={inp.s_q} causal={inp.causal} "
                    f"seqlens={lens} sum_L={int(inp.seqlens.sum())} page=64 cache={cache} seed={seed}",
        "kv_cache": kv,
        "us_per_step": round(us_step, 3),
        "step_mode": "hip_graph" if m["us_step_graph"] is not None else "eager",
        "eager_us_per_step": round(m["us_step_eager"], 3),
        "stage_us": {k: round(v, 3) for k, v in m["median"].items()},
        "stage_us_mean": {k: round(v, 3) for k, v in m["mean"].items()},
        "timed_calls": m["n_ev"],
        "decode_us": round(m["median"]["decode"], 3),
        "latent_kv_TBps": round(work["kv_bytes"] / t_dec / 1e12, 4),
        "decode_TFLOPs": round(tflops, 2),
        "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
        "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFS, 4),
        "roofline": roofline_entry(work, t_dec, traffic),
        "num_slots": m["slots"], "rotating_copies": m["R"],
        "warmup_s": round(m["t_warm"], 3), "warmup_time_steps": m["n_time_warm"],
        "graph_warmup_replays": m["n_graph_warm"],
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    # the GPU reaches its steady clock only after about 100 steps (~15 ms) of
    # load: besides the --warmup steps, untimed steps run for this long first
    # (reported as warmup_s)
    ap.add_argument("--warmup-seconds", type=float, default=0.5)
    ap.add_argument("--config", default="full_heads")
    ap.add_argument("--extra", nargs="*", default=None,
                    help="further workloads measured in the same run and reported under their own keys, "
                         "name or name:fp8 (default with --config full_heads: multi_token, the matrix-bound "
                         "case, and tp_share, the HBM-bound tensor-parallel share, with both caches)")
    ap.add_argument("--kv", choices=("bf16", "fp8"), default="bf16",
                    help="cache format of the main workload: bf16 rows or the quantised page format "
                         "(mla_decode_paged_fp8; at most 32 query rows per sequence)")
    ap.add_argument("--seqlen", type=int, default=0,
                    help="give every sequence of the main workload this length (a length sweep point)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate-plan", action="store_true",
                    help="plan with mla_get_metadata and absorb with mla_absorb_q (two launches) instead of "
                         "mla_absorb_q_with_plan")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the steps as eager launches only (value = eager wall time per step)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed steps, run one plain elementwise copy (torch.neg) of MIB MiB so that "
                         "hardware byte counters can be scaled against a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the library runs on one "
              "GPU and does not shard the decode across GPUs)", file=sys.stderr)
        sys.exit(2)
    extra = args.extra if args.extra is not None else \
        (["multi_token", "tp_share", "tp_share:fp8"] if args.config == "full_heads" else [])

    import torch

    import mla_decode_paged_amd as mla
    from mla_inputs import make_inputs

    torch.cuda.set_device(0)
    mla.load()
    if args.seqlen > 0:
        from mla_inputs import CONFIGS
        inp = make_inputs(args.config, seed=args.seed, seqlens=[args.seqlen] * CONFIGS[args.config]["b"])
    else:
        inp = make_inputs(args.config, seed=args.seed)
    m = measure(mla, inp, args, args.steps, args.warmup, args.warmup_seconds, kv=args.kv)
    append = time_append(mla, inp, m["sets"], args.steps, kv=args.kv)
    del m["sets"]
    if args.copy_calibration > 0:  # reads and writes exactly MIB MiB each
        src = torch.ones((args.copy_calibration << 18,), dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    main_sum = summary(inp, m, recorded_traffic(args.config + ("_fp8" if args.kv == "fp8" else "")) if
                       args.seqlen == 0 else None, args.seed, kv=args.kv)
    us_step = main_sum["us_per_step"]
    line = {
        "metric": METRIC, "value": us_step, "unit": "us/call", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_s": main_sum["warmup_s"], "ms_per_step": round(us_step / 1e3, 6),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": main_sum["workload"], "num_slots": main_sum["num_slots"],
                   "rotating_copies": main_sum["rotating_copies"]},
    }
    for k in ("step_mode", "eager_us_per_step", "stage_us", "stage_us_mean", "timed_calls", "decode_us",
              "latent_kv_TBps", "decode_TFLOPs", "hbm_frac", "mfma_frac", "roofline", "warmup_time_steps",
              "graph_warmup_replays"):
        line[k] = main_sum[k]
    line["append_kv"] = append
    for name in extra:
        torch.cuda.empty_cache()
        cfg_name, _, fmt = name.partition(":")
        fmt = fmt or "bf16"
        xin = make_inputs(cfg_name, seed=args.seed)
        xm = measure(mla, xin, args, args.steps, args.warmup, args.warmup_seconds, kv=fmt)
        del xm["sets"]
        line[name.replace(":", "_")] = summary(xin, xm, recorded_traffic(cfg_name + ("_fp8" if fmt == "fp8" else "")),
                                               args.seed, kv=fmt)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
