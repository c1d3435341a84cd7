#!/usr/bin/env python3
"""Benchmark of the DFlash draft round on one MI355X.

A step is one whole round on one batch of synthetic input already resident in HBM:
fuse the round's new rows (fc + hidden_norm), inject their K/V into every layer's
paged cache, draft one block per stream (non-causal forward + LM-head argmax), and
greedy-verify against a synthetic target row. Every step repeats the same round
(the context length is not advanced), so all steps do identical work.

    python bench.py [--steps K] [--warmup W] [--workload 9b_ctx4k] [--no-cpu-baseline]

Prints one JSON line. `value` is drafted tokens per second (streams x (block - 1)
per round); the line also carries the achieved algorithmic HBM bandwidth of the
round, the roofline of the dominant kernel (per-kernel times from HIP events the
library records around its own launches, in a second timed pass), and the CPU
oracle timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "drafted tokens/sec per draft round + achieved HBM GB/s (9B shape, block 16, 1 GPU)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_TFLOPS = 2500.0      # dense bf16
FP32_TFLOPS = 157.3


def q4_bytes(N, K):
    """Bytes of one weight matrix in the 4-bit packing: per 64 weights of a row, 32 bytes
    of codes and a bf16 scale and bias (rows padded to tiles of 32)."""
    return (N + 31) // 32 * 32 * (K // 64) * 36


def kernel_costs(p, ctx, rows, sampling=False, q4=False):
    """Algorithmic bytes and FLOPs per launch of each kernel of one round.

    Bytes are what the method itself must move: each weight once per call that reads
    it, the tap planes, the stored activations at their storage size (bf16, or fp32
    for fp32 presets) read and written once, context K/V read once over the exact keys
    of each stream's reach. Implementation intermediates (float64 partial sums, chunk
    partials) are not counted.
    """
    es = 4 if p.dtype == "f32" else 2
    h, L, d, I, V, B = p.hidden, p.n_layers, p.head_dim, p.intermediate, p.vocab, p.block_size
    nq, nkv, n = p.n_q_heads * d, p.n_kv_heads * d, p.n_taps
    S = len(ctx)
    R = sum(rows)
    M, Mm = S * B, S * (B - 1)
    k = {}
    k["fuse_fc_gemm"] = dict(bytes=(h * n * h + R * n * h) * es, flops=2 * R * n * h * h)
    k["fuse_rownorm"] = dict(bytes=(R * h + h) * es, flops=3 * R * h)
    k["inject_kv_gemm"] = dict(bytes=(L * 2 * nkv * h + R * h) * es, flops=2 * R * h * L * 2 * nkv)
    k["inject_kv_finish"] = dict(bytes=(L * 2 * R * nkv + L * d) * es, flops=6 * L * R * nkv)
    k["embed"] = dict(bytes=(3 * M * h + h) * es, flops=4 * M * h)
    norm = dict(bytes=(3 * M * h + h) * es, flops=4 * M * h)
    k["norm_in"] = dict(norm, launches=L - 1)
    k["norm_post"] = dict(norm, launches=L)
    k["norm_final"] = dict(bytes=(3 * Mm * h + h) * es, flops=4 * Mm * h)
    k["qkv_gemm"] = dict(bytes=((nq + 2 * nkv) * h + M * h) * es, flops=2 * M * h * (nq + 2 * nkv))
    k["qkv_finish"] = dict(bytes=(M * (nq + 2 * nkv) + 2 * d) * es, flops=8 * M * (nq + nkv))
    for kind, sel in (("attention_full", lambda w: w == 0), ("attention_sliding", lambda w: w > 0)):
        layers = [w for w in p.layer_window[:L] if sel(w)]
        if not layers:
            continue
        wdw = layers[0]
        keys = [min(c, wdw) if wdw > 0 else c for c in ctx]
        k[kind] = dict(bytes=(sum(keys) * 2 * nkv + 2 * M * nq + 2 * M * nkv) * es,
                       flops=sum(4 * p.n_q_heads * B * d * (kk + B) for kk in keys),
                       launches=len(layers))
    k["o_proj_gemm"] = dict(bytes=(h * nq + M * nq) * es, flops=2 * M * nq * h)
    k["gate_up_gemm"] = dict(bytes=(2 * I * h + M * h + M * I) * es, flops=4 * M * h * I)
    k["down_gemm"] = dict(bytes=(h * I + M * I) * es, flops=2 * M * I * h)
    # the sampled round also writes the fp32 logits the draws read
    k["lm_head_gemm"] = dict(bytes=(V * h + Mm * h) * es + (Mm * V * 4 if sampling else 0), flops=2 * Mm * h * V)
    k["argmax_final"] = dict(bytes=Mm * 4, flops=0)
    if sampling:
        # draws: each draft logit row read once; verify: every draft and target row read once
        k["sample_rows"] = dict(bytes=Mm * V * 4 + Mm * 8, flops=0)
        k["verify_sampling"] = dict(bytes=(Mm + M) * V * 4 + (2 * Mm + 3 * S + S * B) * 4, flops=0)
    else:
        k["verify"] = dict(bytes=(S * (B - 1) + S * B) * 4 + (3 * S + S * B) * 4, flops=0)
    if q4:
        # the GEMMs read the 4-bit weights instead of the bf16 ones
        wb = {"fuse_fc_gemm": (h, n * h), "inject_kv_gemm": (L * 2 * nkv, h), "qkv_gemm": (nq + 2 * nkv, h),
              "o_proj_gemm": (h, nq), "gate_up_gemm": (2 * I, h), "down_gemm": (h, I), "lm_head_gemm": (V, h)}
        for name, (N_, K_) in wb.items():
            k[name]["bytes"] += q4_bytes(N_, K_) - N_ * K_ * es
    for name in ("qkv_gemm", "qkv_finish", "o_proj_gemm", "gate_up_gemm", "down_gemm"):
        k[name]["launches"] = L
    for name, v in k.items():
        v.setdefault("launches", 1)
    return k


# Source files whose kernels a committed traffic measurement covers, per kernel name.
_GEMM_SOURCES = ["gemm.hip", "gemm_tall.hip", "common.hpp", "kernels.h"]
KERNEL_SOURCES = {
    "gate_up_gemm": _GEMM_SOURCES,
    "lm_head_gemm": _GEMM_SOURCES,
    "down_gemm": _GEMM_SOURCES,
    "qkv_gemm": _GEMM_SOURCES,
    "o_proj_gemm": _GEMM_SOURCES,
    "fuse_fc_gemm": _GEMM_SOURCES,
    "inject_kv_gemm": _GEMM_SOURCES,
    "attention_full": ["attention.hip", "common.hpp", "kernels.h"],
    "attention_sliding": ["attention.hip", "common.hpp", "kernels.h"],
}
COPY_CALIBRATION_BYTES = 256 << 20


def sources_digest(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(ROOT, "block_diffusion_drafter_dflash_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed PMC measurement, or None when
    there is none for this kernel and workload or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    for r in rec.get("kernels", []):
        if r.get("kernel") == kernel and r.get("workload") == workload and r.get("sources_sha256") == sources_digest(kernel):
            return int(r["fetch_bytes"] + r["write_bytes"])
    return None


def copy_calibration():
    """One plain copy-like kernel of known traffic (reads and writes COPY_CALIBRATION_BYTES),
    outside every timed region, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = COPY_CALIBRATION_BYTES // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def round_totals(costs):
    b = sum(v["bytes"] * v["launches"] for v in costs.values())
    f = sum(v["flops"] * v["launches"] for v in costs.values())
    return b, f


def host_cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(case, sample_streams, min_seconds=10.0):
    """The oracle, as it stands, on whole rounds of the chosen streams, repeated until
    at least min_seconds of CPU work have been timed."""
    from oracle import dflash_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    W = case.weights_np()
    streams = case.oracle_streams(sample_streams)
    for st in streams:   # an existing context built from taps is set-up, outside the timed rounds
        if "ctx_taps" in st:
            st["k_ctx"], st["v_ctx"] = O.context_from_taps(case.p, st.pop("ctx_taps"), W)
    reps, total, out = 0, 0.0, None
    while total < min_seconds:
        t0 = time.perf_counter()
        out = O.run_round(case.p, W, streams)
        total += time.perf_counter() - t0
        reps += 1
    dt = total / reps
    drafted = len(sample_streams) * (case.p.block_size - 1)
    return dict(value=round(drafted / dt, 3), unit="drafted tokens/s", cores=int(threads), kind="oracle",
                cpu_model=host_cpu_model(), host_threads=os.cpu_count(),
                sample=f"{reps} whole rounds (fuse {sum(case.rows[s] for s in sample_streams)} rows, inject, "
                       f"draft) of stream(s) {sample_streams} of the same workload, float64 numpy; "
                       f"{dt:.2f} s per round", seconds=round(total, 2)), out


def graph_replay(torch, step, st, steps):
    """ms per round when one round is captured into a HIP graph and replayed `steps`
    times on stream `st` (the library allocates nothing and clears with kernels, so
    a round captures as it runs). A capture failure is reported, not raised."""
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(st)
        with torch.cuda.stream(side):
            step()
        st.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(steps):
            g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        return {"ms_per_step": round(e0.elapsed_time(e1) / steps, 5), "replays": steps}
    except RuntimeError as exc:
        return {"error": str(exc)[:200]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="9b_ctx4k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-steps", type=int, default=20)
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay pass")
    ap.add_argument("--defer", action="store_true",
                    help="with --prefill: inject each prompt row only into the layers that will read it")
    ap.add_argument("--q4", action="store_true",
                    help="the drafter's 4-bit weights (groups of 64) instead of bf16 (a separate workload)")
    ap.add_argument("--prefill", type=int, default=0,
                    help="instead of the round: fuse + inject this many prompt rows of one stream")
    ap.add_argument("--sampling", type=float, default=0.0,
                    help="temperature T > 0: the round drafts by sampling and verifies by speculative sampling "
                         "(draft logits written, tempered draws, synthetic target logits)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the round shards by "
              f"streams with no exchange, so N GPUs run N independent copies).", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as wl
    from workloads.round_case import RoundCase

    torch.cuda.init()
    p = wl.preset(args.workload)
    if args.prefill > 0:
        prefill_main(args, p)
        return
    print(f"[bench] workload {p.name}{' (4-bit weights)' if args.q4 else ''}: setting up", file=sys.stderr, flush=True)
    case = RoundCase(p, q4=args.q4)
    S, B = p.n_streams, p.block_size

    # target row from an untimed round of the same inputs
    case.run_gpu()
    case.set_target_from(case.draft.cpu().numpy())
    torch.cuda.synchronize()

    if args.sampling > 0:
        # sampled round: the draft's logits are written, each mask row is drawn from its
        # tempered softmax, and the block is verified by speculative sampling against
        # seeded target logits (what a target model would return for the block)
        T = args.sampling
        g = torch.Generator(device="cuda").manual_seed(p.seed + 17)
        target_logits = torch.randn((S, B, p.vocab), generator=g, device="cuda") * 2.0
        u_draw = torch.rand(S * (B - 1), generator=g, device="cuda")
        u_acc = torch.rand((S, B - 1), generator=g, device="cuda")
        u_smp = torch.rand(S, generator=g, device="cuda")
        s_draft = torch.zeros(S * (B - 1), dtype=torch.int32, device="cuda")
        s_token = torch.zeros(S, dtype=torch.int32, device="cuda")

        def step():
            case.fuse()
            case.inject()
            case.draft_block(logits=True, top2=False)
            case.dr.dflash_sample_rows(case.logits.view(S * (B - 1), p.vocab), T, u_draw, s_draft, case.ws)
            case.dr.dflash_verify_sampling(s_draft.view(S, B - 1), case.logits, target_logits, T, u_acc, u_smp,
                                           case.accept, s_token, case.committed, case.ws)
    else:
        def step():
            case.fuse()
            case.inject()
            case.draft_block(logits=False, top2=False)
            case.verify()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done; timing {args.steps} steps", file=sys.stderr, flush=True)
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(st)
    for _ in range(args.steps):
        step()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = e0.elapsed_time(e1) / args.steps

    # distribution of single rounds (a separate pass; the timed region above is untouched)
    qn = min(args.steps, 50)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(qn)]
    for a, b in evs:
        a.record(st)
        step()
        b.record(st)
    torch.cuda.synchronize()
    per_round = sorted(a.elapsed_time(b) for a, b in evs)
    quant = {q: round(per_round[min(qn - 1, int(f * (qn - 1) + 0.5))], 5)
             for q, f in (("p10", 0.1), ("p50", 0.5), ("p90", 0.9))}

    # per-kernel pass: the library brackets each of its launches with events on this stream
    case.dr.set_profiling(True)
    case.dr.profile_read()
    for _ in range(args.profile_steps):
        step()
    torch.cuda.synchronize()
    prof = case.dr.profile_read()
    case.dr.set_profiling(False)
    print(f"[bench] timed {ms:.4f} ms/step; per-kernel pass done", file=sys.stderr, flush=True)

    # the same round captured once as a HIP graph and replayed (reported beside the
    # eager figure, which stays the headline)
    graph = None if args.no_graph else graph_replay(torch, step, st, args.steps)

    costs = kernel_costs(p, case.ctx, case.rows, sampling=args.sampling > 0, q4=args.q4)
    tot_bytes, tot_flops = round_totals(costs)
    drafted = S * (B - 1)
    value = drafted / (ms * 1e-3)
    kernels = {}
    for name, (cnt, total) in prof.items():
        per = total / cnt
        c = costs.get(name, {"bytes": 0, "flops": 0})
        kernels[name] = dict(launches_per_step=cnt / args.profile_steps, avg_ms=per,
                             ms_per_step=total / args.profile_steps,
                             gbps=c["bytes"] / (per * 1e-3) / 1e9 if per > 0 else None,
                             tflops=c["flops"] / (per * 1e-3) / 1e12 if per > 0 else None)
    dom = max(kernels, key=lambda n: kernels[n]["ms_per_step"])
    kd = kernels[dom]
    mfma_dtype_peak = FP32_TFLOPS if p.dtype == "f32" else MFMA_BF16_TFLOPS
    ai = costs[dom]["flops"] / max(1, costs[dom]["bytes"])
    if ai * HBM_PEAK_GBS * 1e9 < mfma_dtype_peak * 1e12:
        roof = dict(bound="hbm", achieved=round(kd["gbps"], 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(kd["gbps"] / HBM_PEAK_GBS, 4))
    else:
        roof = dict(bound="mfma", achieved=round(kd["tflops"], 2), peak=mfma_dtype_peak, unit="TFLOP/s",
                    frac=round(kd["tflops"] / mfma_dtype_peak, 4))
    roof.update(kernel=dom, bytes_per_launch=costs[dom]["bytes"], flops_per_launch=costs[dom]["flops"],
                avg_launch_ms=round(kd["avg_ms"], 5), traffic=measured_traffic(dom, p.name))

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "drafted tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": p.dtype, "data": "synthetic",
        "config": {"workload": (p.note or p.name) + (f", sampled at T={args.sampling}" if args.sampling > 0 else "")
                   + (", 4-bit drafter weights (groups of 64)" if args.q4 else ""),
                   "preset": p.name, "streams": S, "block": B,
                   "context": case.ctx if S > 1 else case.ctx[0], "rows_fused": case.R,
                   "hidden": p.hidden, "layers": p.n_layers, "vocab": p.vocab},
        "hbm_gbps": round(tot_bytes / (ms * 1e-3) / 1e9, 1),
        "hbm_frac_of_peak": round(tot_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "mfma_frac_of_peak": round(tot_flops / (ms * 1e-3) / 1e12 / mfma_dtype_peak, 5),
        "round_bytes": tot_bytes, "round_flops": tot_flops, "wall_s_timed": round(wall, 4),
        "round_ms_quantiles": quant,
        "graph_replay": graph,
        "bytes_per_drafted_token": round(tot_bytes / drafted),
        "bytes_per_accepted_token": round(tot_bytes / max(1, case.R)),
        "roofline": roof,
        "kernels": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in sorted(kernels.items(), key=lambda kv: -kv[1]["ms_per_step"])},
    }
    copy_calibration()
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline (one round)", file=sys.stderr, flush=True)
        sample = [0] if S == 1 else [int(min(range(S), key=lambda s: case.ctx[s]))]
        cb, _ = cpu_baseline(case, sample)
        out["cpu_baseline"] = cb
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def prefill_main(args, p):
    """Fuse + inject of `args.prefill` prompt rows of one stream at the workload's shapes
    (the step before the round at prompt scale): rows/s, the fc GEMM against the MFMA
    roofline, and the oracle on a few of the rows."""
    import torch
    import workloads as wl
    from workloads.round_case import RoundCase, to_np

    R = args.prefill
    from workloads.presets import small_variant
    q = small_variant(p, n_streams=1)
    print(f"[bench] prefill: {R} rows at {p.name} shapes: setting up", file=sys.stderr, flush=True)
    case = RoundCase(q, ctx=[max(R, 4096)], rows=[R])
    st = torch.cuda.current_stream()

    groups = None
    if args.defer:
        # layers reading each prompt row at the prompt length; the masks only grow with
        # the position, so each mask's rows are one contiguous range
        P = case.ctx[0]
        pos = case.row_pos.cpu().tolist()
        masks = [case.dr.dflash_layers_reading(x, P) for x in pos]
        groups, a = [], 0
        for i in range(1, len(masks) + 1):
            if i == len(masks) or masks[i] != masks[a]:
                groups.append((a, i, masks[a]))
                a = i
        assert all(g[2] & masks[-1] == g[2] for g in groups)
        print(f"[bench] deferred inject: {[(b - a, bin(m)) for a, b, m in groups]}", file=sys.stderr, flush=True)

    def step():
        case.fuse()
        if groups is None:
            case.inject()
        else:
            for a, b, m in groups:
                case.dr.dflash_inject_kv_layers(case.fused[a:b], case.row_stream[a:b], case.row_pos[a:b], case.kv, m,
                                                case.ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(args.steps):
        step()
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    case.dr.set_profiling(True)
    case.dr.profile_read()
    for _ in range(args.profile_steps):
        step()
    torch.cuda.synchronize()
    prof = case.dr.profile_read()
    case.dr.set_profiling(False)

    costs = kernel_costs(q, case.ctx, case.rows)
    if groups is not None:
        # each call reads its selected layers' weights and its rows, and computes their K/V
        es = 4 if q.dtype == "f32" else 2
        nkv, h, d = q.n_kv_heads * q.head_dim, q.hidden, q.head_dim
        gb = gf = fb = ff = 0
        for a, b, m in groups:
            nl, r = bin(m).count("1"), b - a
            gb += (nl * 2 * nkv * h + r * h) * es
            gf += 2 * r * h * nl * 2 * nkv
            fb += (nl * 2 * r * nkv + nl * d) * es
            ff += 6 * nl * r * nkv
        ng = len(groups)   # per launch: the average over the calls of a step
        costs["inject_kv_gemm"] = dict(costs["inject_kv_gemm"], bytes=gb / ng, flops=gf / ng, launches=ng)
        costs["inject_kv_finish"] = dict(costs["inject_kv_finish"], bytes=fb / ng, flops=ff / ng, launches=ng)
    names = ("fuse_fc_gemm", "fuse_rownorm", "inject_kv_gemm", "inject_kv_finish")
    tot_bytes = sum(costs[n]["bytes"] * costs[n].get("launches", 1) for n in names)
    tot_flops = sum(costs[n]["flops"] * costs[n].get("launches", 1) for n in names)
    kernels = {}
    for name, (cnt, total) in prof.items():
        per = total / cnt
        c = costs.get(name, {"bytes": 0, "flops": 0})
        kernels[name] = dict(launches_per_step=cnt / args.profile_steps, avg_ms=round(per, 5),
                             gbps=round(c["bytes"] / (per * 1e-3) / 1e9, 1),
                             tflops=round(c["flops"] / (per * 1e-3) / 1e12, 2))
    dom = "fuse_fc_gemm"
    peak = FP32_TFLOPS if q.dtype == "f32" else MFMA_BF16_TFLOPS
    roof = dict(bound="mfma", achieved=kernels[dom]["tflops"], peak=peak, unit="TFLOP/s",
                frac=round(kernels[dom]["tflops"] / peak, 4), kernel=dom,
                bytes_per_launch=costs[dom]["bytes"], flops_per_launch=costs[dom]["flops"],
                avg_launch_ms=kernels[dom]["avg_ms"], traffic=None)
    out = {
        "metric": ("prefill-scale fuse + inject: prompt rows/s (fc GEMM + hidden norm + K/V of "
                   + ("the layers that read each row)" if groups is not None else "every layer)")),
        "value": round(R / (ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": q.dtype, "data": "synthetic",
        "config": {"workload": f"fuse + {'deferred ' if groups is not None else ''}inject of {R} prompt rows at "
                               f"{p.name} shapes", "preset": p.name,
                   "rows": R, "hidden": q.hidden, "taps": q.n_taps, "layers": q.n_layers},
        "mfma_frac_of_peak": round(tot_flops / (ms * 1e-3) / 1e12 / peak, 4),
        "hbm_gbps": round(tot_bytes / (ms * 1e-3) / 1e9, 1), "step_bytes": tot_bytes, "step_flops": tot_flops,
        "roofline": roof, "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        from oracle import dflash_oracle as O
        W = case.weights_np()
        idx = list(range(0, R, max(1, R // 8)))[:8]
        taps = [to_np(t[idx]) for t in case.taps]
        reps, total = 0, 0.0
        while total < 10.0:
            t0 = time.perf_counter()
            f = O.fuse_taps(q, taps, W)
            O.inject_kv(q, f, [case.ctx[0] - R + i for i in idx], W)
            total += time.perf_counter() - t0
            reps += 1
        per_row = total / reps / len(idx)
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:  # pragma: no cover
            threads = os.cpu_count() or 1
        out["cpu_baseline"] = dict(value=round(1.0 / per_row, 2), unit="rows/s", cores=int(threads), kind="oracle",
                                   cpu_model=host_cpu_model(),
                                   sample=f"{reps} x fuse + inject of {len(idx)} of the {R} rows, float64 numpy",
                                   seconds=round(total, 2))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
