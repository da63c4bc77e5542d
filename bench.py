"""Benchmark: one forward pass of the Qwen3-30B-A3B-shaped MoE layer per step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload qwen3_prefill]

A step is the whole layer (route, permute, grouped gate/up, grouped down,
shared expert when present, combine, stats) on T tokens already resident in
HBM, enqueued on one stream through the C ABI of libmoe.so.  K steps are timed
with HIP events between two device synchronizations.  Prints one JSON line:
tokens/s, the roofline of the dominant kernel (the grouped gate/up GEMM, timed
with events on its own stream around each launch), the grouped-GEMM share of
the bf16 MFMA peak, the decode-regime layer against HBM bandwidth, and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_CLOCK_GHZ = 2.4
PEAK_BF16_FLOPS = 256 * 4096 * PEAK_CLOCK_GHZ * 1e9  # dense bf16 MFMA: 256 CUs x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_BYTES = 8.0e12                   # HBM3E
# The headline steps' untimed warm-up runs at least this long (W steps, then more
# if W steps take less): the clock settles under load in tens of milliseconds.
HEADLINE_MIN_WARM_MS = 200.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="qwen3_prefill")
    p.add_argument("--decode-workload", default="qwen3_decode")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the CPU baseline")
    p.add_argument("--configs", action="store_true",
                   help="instead of the headline line, time the whole layer on every configured shape "
                        "(one JSON line per shape; generating the largest weight set takes a while)")
    p.add_argument("--combine-compare", default="", metavar="W1,W2,...",
                   help="time the gather and the scatter combine on these workloads")
    p.add_argument("--sweep-tokens", default="", metavar="T1,T2,...",
                   help="instead of the headline line, time the --workload layer at each token count "
                        "(same weights; one JSON line each)")
    p.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                   help="only copy BYTES bytes device to device three times (a plain copy kernel of known size "
                        "that scales the HBM byte counters) and exit")
    return p.parse_args()


# The gate/up GEMM's HBM bytes per launch come from rocprofv3 counter runs recorded in
# this summary, together with a hash of the kernel sources they were taken on; they
# are reported only while the sources are unchanged.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gate_up_gemm_qwen3_prefill_pmc.txt")
CLOCK_SUMMARY = os.path.join(ROOT, "profiles", "grouped_gemm_qwen3_prefill_mfma_l2.txt")
GEMM_SOURCES = ("mixture_experts_ffn_08_amd/csrc/grouped_gemm.hip", "mixture_experts_ffn_08_amd/csrc/common.h",
                "mixture_experts_ffn_08_amd/csrc/kernels.h")


def gemm_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per gate/up launch from the counter summary, or None if there is
    none or the kernel sources changed since it was taken."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    fields = {}
    with open(TRAFFIC_SUMMARY) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                key, _, val = line.partition("=")
                fields[key.strip()] = val.strip()
    if fields.get("kernel_source_sha256") != gemm_source_hash():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def recorded_clocks():
    """Sustained clocks (GHz) of the gate/up and down launches from the counter
    summary, or None if there is none or the kernel sources changed since."""
    if not os.path.exists(CLOCK_SUMMARY):
        return None
    fields = {}
    with open(CLOCK_SUMMARY) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                key, _, val = line.partition("=")
                fields[key.strip()] = val.strip()
    if fields.get("kernel_source_sha256") != gemm_source_hash():
        return None
    try:
        return float(fields["gate_up_clock_ghz"]), float(fields["down_clock_ghz"])
    except (KeyError, ValueError):
        return None


def copy_probe(nbytes: int):
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes}), flush=True)


def measured_copy_rate(torch, nbytes: int = 1 << 30) -> float:
    """Bytes moved per second (read + write) by a plain device-to-device copy of
    nbytes: what streaming through HBM reaches on this part, beside the spec."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    rate = 2.0 * nbytes / (e0.elapsed_time(e1) / 10 * 1e-3)
    del src, dst
    torch.cuda.empty_cache()
    return rate


def timed_steps(layer, x, bufs, steps, warmup, stream, torch, min_warm_ms=0.0):
    """Run warmup + timed steps; returns (ms per step, per-launch ms of gate/up, down (with
    the scatter combine: down and combine) and the shared expert (0 without one)).
    With large groups the balance statistics run on a second stream beside the
    combine (MoeLayer.forward); a step ends when both streams are done.  The timed
    steps record no events inside; the per-launch GEMM times come from as many
    further steps with events around the two launches.  min_warm_ms > 0 (the
    sweeps): further warm-up steps until the warm-up has run that long, since the
    part takes tens of milliseconds of load to reach its working clock and a
    small layer's warm-up steps may not add up to that.  The warm-up's duration is
    left in timed_steps.warm_ms."""
    side = torch.cuda.Stream()

    def step(ev=None):
        layer.forward(x, bufs, stream, side_stream=side, marks=ev)

    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0.record(stream)
    for _ in range(warmup):
        step()
    w1.record(stream)
    torch.cuda.synchronize()
    spent = w0.elapsed_time(w1)
    while warmup > 0 and min_warm_ms > spent:
        # the first steps run cold and slow: estimate from the last batch, and repeat
        batch = max(warmup, 1)
        w0.record(stream)
        for _ in range(batch):
            step()
        w1.record(stream)
        torch.cuda.synchronize()
        last = w0.elapsed_time(w1)
        spent += last
        warmup = max(1, int(np.ceil((min_warm_ms - spent) / max(last / batch, 1e-3))))
    timed_steps.warm_ms = spent
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    total = start.elapsed_time(end)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    gu = [e[0].elapsed_time(e[1]) for e in evs]
    dn = [e[1].elapsed_time(e[2]) for e in evs]
    sh = [e[2].elapsed_time(e[3]) for e in evs]
    if getattr(layer, "scatter_combine", False):
        dn, sh = sh, dn  # the shared expert runs before the down GEMM with the combine
    return total / steps, float(np.mean(gu)), float(np.mean(dn)), float(np.mean(sh))


def cpu_baseline(inp, target_s):
    """The oracle, as it stands, on a growing prefix of the workload's tokens until
    it has run for about target_s seconds; tokens/s of the last sample, with the
    oracle's own per-step wall times.  `cores` is the number of threads the oracle
    ran on (its matrix products run in the BLAS library's thread pool; the rest
    is one thread); `cpu_count` is what the operating system reports."""
    import oracle
    from mixture_experts_ffn_08_amd import inputs as minp

    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] + [1])
    except Exception:  # pragma: no cover
        blas = 1
    s = inp.shape
    ex = {}

    def weights(e):
        if e not in ex:
            ex[e] = tuple(minp.as_f32(m, s.dtype) for m in inp.expert(e))
        return ex[e]

    for e in range(s.E):
        weights(e)
    sh = inp.shared()
    sh = None if sh is None else tuple(minp.as_f32(m, s.dtype) for m in sh)
    xs = minp.as_f32(inp.x, s.dtype)
    wr = minp.as_f32(inp.w_router, s.dtype)
    n, elapsed = 64, 0.0
    while True:
        n = min(n, s.T)
        stages = {}
        t0 = time.perf_counter()
        oracle.layer_forward(xs[:n], wr, inp.bias, weights, sh, k=s.k, mode=s.mode, renorm=s.renorm, phi=s.phi,
                             alpha=s.alpha, dtype=s.dtype, timings=stages)
        elapsed = time.perf_counter() - t0
        if elapsed >= target_s or n == s.T:
            break
        n = int(n * min(8.0, max(1.5, 1.1 * target_s / max(elapsed, 1e-3))))
    return {"value": n / elapsed, "unit": "tokens/s", "cores": int(blas), "kind": "oracle",
            "sample": f"first {n} of {s.T} tokens of the {s.name} layer, the whole oracle forward "
                      f"(float64 products of the bf16 values, numpy/BLAS), {elapsed:.1f} s",
            "cpu_count": os.cpu_count(), "blas_threads": int(blas),
            "stage_s": {k: round(v, 4) for k, v in stages.items()}}


def ep_share(weights, x, bufs, shape, stream, torch, gpus: int = 8, phi: float = 1.25, steps: int = 20):
    """One GPU's share of the layer under expert parallelism over `gpus` GPUs: the
    first E / gpus experts, each with C = ceil(phi k T / E) slots of the
    capacity-padded layout (the fixed-size buffers an all-to-all exchange would
    deliver; the exchange itself is not run).  Rows are the dispatch of the
    layer's own routing (bufs.topk_idx); the GEMMs run over all G C slots,
    padding included.  Returns the gate/up and down launch times and their MFMA
    fractions, counting either the kept rows or every slot."""
    from mixture_experts_ffn_08_amd import _lib
    s = shape
    C = _lib.moe_capacity(s.T, s.k, s.E, phi)
    G = s.E // gpus
    dev = x.device
    i32 = torch.int32
    counts = torch.empty(s.E, dtype=i32, device=dev)
    offsets = torch.empty(s.E + 1, dtype=i32, device=dev)
    row_of = torch.empty((s.T, s.k), dtype=i32, device=dev)
    slot_token = torch.empty(s.E * C, dtype=i32, device=dev)
    x_slots = torch.empty((s.E * C, s.d), dtype=x.dtype, device=dev)
    ws = torch.empty(max(_lib.moe_permute_workspace_bytes(s.T, s.k, s.E), 1), dtype=torch.uint8, device=dev)
    _lib.moe_permute_padded(bufs.topk_idx, s.T, s.k, s.E, C, x, s.d, counts, offsets, row_of, slot_token, x_slots,
                            ws, stream)
    rows = G * C
    xs, off = x_slots[:rows], offsets[:G + 1]
    a = torch.empty((rows, s.F), dtype=x.dtype, device=dev)
    y = torch.empty((rows, s.d), dtype=x.dtype, device=dev)
    gate, up, down = weights.gate[:G], weights.up[:G], weights.down[:G]

    def run(ev=None):
        if ev is not None:
            ev[0].record(stream)
        _lib.moe_grouped_gate_up(xs, None, 0, off, G, rows, s.d, s.F, gate, up, a, stream)
        if ev is not None:
            ev[1].record(stream)
        _lib.moe_grouped_down(a, off, G, rows, s.F, s.d, down, y, stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(steps):
        run()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in evs:
        run(e)
    torch.cuda.synchronize()
    gu = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    dn = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    kept = int(torch.clamp(counts[:G], max=C).sum().item())
    f_kept, f_all = 6.0 * kept * s.d * s.F, 6.0 * rows * s.d * s.F
    t = (gu + dn) * 1e-3
    return {"workload": f"{s.name} expert-parallel share: experts 0..{G - 1} of {s.E} ({gpus} GPUs), "
                        f"capacity-padded layout, C = {C} (phi = {phi})",
            "experts": G, "capacity": C, "slots": rows, "kept_rows": kept, "gate_up_ms": gu, "down_ms": dn,
            "tflops_all_slots": f_all / t / 1e12, "frac_of_mfma_peak_all_slots": f_all / t / PEAK_BF16_FLOPS,
            "tflops_kept_rows": f_kept / t / 1e12, "frac_of_mfma_peak_kept_rows": f_kept / t / PEAK_BF16_FLOPS}


def config_sweep(steps: int, warmup: int):
    """Time the layer on every configured shape (synthetic inputs, seed 0): one
    JSON line each with tokens/s, the routed and shared expert FLOPs against the
    bf16 MFMA peak, the algorithmic bytes against HBM, and (prefill shapes) one
    GPU's share of the layer under 8-way expert parallelism."""
    import torch

    from mixture_experts_ffn_08_amd import inputs as minp
    from mixture_experts_ffn_08_amd.layer import Buffers, DeviceWeights, MoeLayer, to_device

    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    for name in ("mixtral", "mixtral_cap", "qwen2", "qwen3_prefill", "qwen3_decode", "dsv3_skew"):
        shape = minp.SHAPES[name]
        t0 = time.time()
        inp = minp.LayerInputs(shape, seed=0)
        weights = DeviceWeights(inp, "cuda:0")
        layer = MoeLayer(weights)
        x = to_device(inp.x, shape.dtype, "cuda:0")
        bufs = Buffers(shape, shape.T, "cuda:0")
        setup_s = time.time() - t0
        with torch.cuda.stream(stream):
            ms, gu_ms, dn_ms, sh_ms = timed_steps(layer, x, bufs, steps, warmup, stream, torch, min_warm_ms=150.0)
        R = int(bufs.offsets[-1].item())
        touched = int((bufs.counts > 0).sum().item())
        s = shape
        # one GPU's share under 8-way expert parallelism, on this layer's own routing
        with torch.cuda.stream(stream):
            eps = ep_share(weights, x, bufs, shape, stream, torch) if s.T >= 1024 and s.E >= 8 else None
        routed_flops = 6.0 * R * s.d * s.F
        shared_flops = 6.0 * s.T * s.d * s.F_shared
        flops = routed_flops + shared_flops + 2.0 * s.T * s.d * s.E
        nbytes = (touched * 3 * s.d * s.F + 3 * s.d * s.F_shared + s.E * s.d + 2 * s.T * s.d) * s.elem_bytes
        print(json.dumps({
            "workload": name, "T": s.T, "d": s.d, "E": s.E, "k": s.k, "F": s.F, "F_shared": s.F_shared,
            "capacity_factor": s.phi, "ms_per_step": ms, "tokens_per_s": s.T / (ms * 1e-3),
            "gate_up_ms": gu_ms, "down_ms": dn_ms,
            "routed_gemm_frac_of_mfma_peak": routed_flops / ((gu_ms + dn_ms) * 1e-3) / PEAK_BF16_FLOPS,
            "shared_ms": sh_ms if s.F_shared else None,
            "shared_tflops": shared_flops / (sh_ms * 1e-3) / 1e12 if s.F_shared else None,
            "shared_frac_of_mfma_peak": shared_flops / (sh_ms * 1e-3) / PEAK_BF16_FLOPS if s.F_shared else None,
            "kept_assignments": R, "experts_touched": touched,
            "max_over_mean": float(bufs.max_over_mean.item()),
            "layer_tflops": flops / (ms * 1e-3) / 1e12, "frac_of_mfma_peak": flops / (ms * 1e-3) / PEAK_BF16_FLOPS,
            "algorithmic_bytes": nbytes, "hbm_frac": nbytes / (ms * 1e-3) / PEAK_HBM_BYTES,
            "ep_share": eps, "steps": steps, "warmup": warmup, "setup_s": round(setup_s, 1)}), flush=True)
        del weights, layer, x, bufs, inp
        torch.cuda.empty_cache()


def combine_compare(names, steps: int, warmup: int, rounds: int = 3):
    """The layer with the gather combine (the down GEMM writes y_perm, a second
    kernel sums each token's rows in slot order) against the scatter combine (the
    down GEMM adds its weighted rows into a float32 accumulator with atomics, then
    one pass adds the shared expert and rounds).  Same weights and inputs; the two
    forms are timed in alternation, `rounds` times each, and the median kept.  One
    JSON line per workload: whole-step times, and the down launch alone (gather)
    against the down-with-combine call (scatter)."""
    import torch

    from mixture_experts_ffn_08_amd import inputs as minp
    from mixture_experts_ffn_08_amd.layer import Buffers, DeviceWeights, MoeLayer, to_device

    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    for name in names:
        shape = minp.SHAPES[name]
        inp = minp.LayerInputs(shape, seed=0)
        weights = DeviceWeights(inp, "cuda:0")
        x = to_device(inp.x, shape.dtype, "cuda:0")
        forms = {"gather": MoeLayer(weights), "scatter": MoeLayer(weights, scatter_combine=True)}
        bufs = {k: Buffers(shape, shape.T, "cuda:0", scatter=(k == "scatter")) for k in forms}
        res = {k: [] for k in forms}
        with torch.cuda.stream(stream):
            for r in range(rounds):
                for k, lay in forms.items():
                    ms, gu, dn, sh = timed_steps(lay, x, bufs[k], steps, warmup, stream, torch, min_warm_ms=150.0)
                    res[k].append((ms, gu, dn, sh))
        med = {k: np.median(np.array(v), axis=0) for k, v in res.items()}
        y_diff = float((bufs["gather"].y.float() - bufs["scatter"].y.float()).abs().max().item())
        print(json.dumps({
            "workload": name, "T": shape.T, "d": shape.d, "E": shape.E, "k": shape.k,
            "gather_ms_per_step": float(med["gather"][0]), "scatter_ms_per_step": float(med["scatter"][0]),
            "scatter_speedup": float(med["gather"][0] / med["scatter"][0]),
            "gather_down_ms": float(med["gather"][2]),
            "scatter_down_combine_ms": float(med["scatter"][2]),
            "gather_steps_ms_all": [round(v[0], 4) for v in res["gather"]],
            "scatter_steps_ms_all": [round(v[0], 4) for v in res["scatter"]],
            "max_abs_y_diff": y_diff, "steps": steps, "warmup": warmup, "rounds": rounds}), flush=True)
        del weights, x, forms, bufs, inp
        torch.cuda.empty_cache()


def token_sweep(name: str, tokens, steps: int, warmup: int):
    """The layer of workload `name` at other token counts, on one set of weights:
    ms per step, the two GEMM launches, and the touched experts' weight bytes
    against the step time and against 8 TB/s."""
    import torch

    from mixture_experts_ffn_08_amd import inputs as minp
    from mixture_experts_ffn_08_amd.layer import Buffers, DeviceWeights, MoeLayer, to_device

    torch.cuda.set_device(0)
    base = minp.SHAPES[name]
    weights = DeviceWeights(minp.LayerInputs(base, seed=0), "cuda:0")
    stream = torch.cuda.Stream()
    for T in tokens:
        s = base.with_(T=T, name=f"{name}_T{T}")
        inp = minp.LayerInputs(s, seed=0)
        layer = MoeLayer(weights)
        layer.shape = s
        x = to_device(inp.x, s.dtype, "cuda:0")
        bufs = Buffers(s, T, "cuda:0")
        with torch.cuda.stream(stream):
            ms, gu_ms, dn_ms, _ = timed_steps(layer, x, bufs, steps, warmup, stream, torch, min_warm_ms=150.0)
        touched = int((bufs.counts > 0).sum().item())
        wbytes = touched * 3 * s.d * s.F * s.elem_bytes
        nbytes = wbytes + (s.E * s.d + 2 * T * s.d) * s.elem_bytes
        print(json.dumps({"workload": s.name, "T": T, "rows_per_expert": T * s.k / s.E, "ms_per_step": ms,
                          "tokens_per_s": T / (ms * 1e-3), "gate_up_ms": gu_ms, "down_ms": dn_ms,
                          "experts_touched": touched, "algorithmic_bytes": nbytes,
                          "hbm_frac": nbytes / (ms * 1e-3) / PEAK_HBM_BYTES,
                          "gemm_weight_stream_frac": wbytes / ((gu_ms + dn_ms) * 1e-3) / PEAK_HBM_BYTES,
                          "steps": steps, "warmup": warmup}), flush=True)
        del x, bufs, layer
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.configs:
        config_sweep(args.steps, args.warmup)
        return
    if args.combine_compare:
        combine_compare(args.combine_compare.split(","), args.steps, args.warmup)
        return
    if args.sweep_tokens:
        token_sweep(args.workload, [int(v) for v in args.sweep_tokens.split(",")], args.steps, args.warmup)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(there is no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch

    from mixture_experts_ffn_08_amd import inputs as minp
    from mixture_experts_ffn_08_amd.layer import Buffers, DeviceWeights, MoeLayer, to_device

    torch.cuda.set_device(0)
    shape = minp.SHAPES[args.workload]
    inp = minp.LayerInputs(shape, seed=0)
    weights = DeviceWeights(inp, "cuda:0")
    layer = MoeLayer(weights)
    x = to_device(inp.x, shape.dtype, "cuda:0")
    bufs = Buffers(shape, shape.T, "cuda:0")
    stream = torch.cuda.Stream()
    # The other legs run first: the part takes tens of milliseconds of load to
    # reach its working clock, so the headline steps are timed on a busy device
    # (and their own warm-up runs for at least HEADLINE_MIN_WARM_MS).
    extra = {}
    # decode regime on the same weights
    if args.decode_workload:
        dshape = minp.SHAPES[args.decode_workload]
        assert (dshape.d, dshape.E, dshape.F, dshape.k) == (shape.d, shape.E, shape.F, shape.k)
        dinp = minp.LayerInputs(dshape, seed=0)
        dlayer = MoeLayer(weights)
        dlayer.shape = dshape
        dx = to_device(dinp.x, dshape.dtype, "cuda:0")
        dbufs = Buffers(dshape, dshape.T, "cuda:0")
        with torch.cuda.stream(stream):
            dms, _, _, _ = timed_steps(dlayer, dx, dbufs, max(args.steps, 50), args.warmup, stream, torch,
                                       min_warm_ms=150.0)
        touched = int((dbufs.counts > 0).sum().item())
        dbytes = (touched * 3 * dshape.d * dshape.F + dshape.E * dshape.d + 2 * dshape.T * dshape.d) * 2
        copy_rate = measured_copy_rate(torch)
        extra["decode"] = {"workload": f"{dshape.name}: T={dshape.T}", "tokens_per_s": dshape.T / (dms * 1e-3),
                           "ms_per_step": dms, "experts_touched": touched, "algorithmic_bytes": dbytes,
                           "hbm_frac": dbytes / (dms * 1e-3) / PEAK_HBM_BYTES,
                           "measured_copy_TBps": copy_rate / 1e12,
                           "frac_of_measured_copy": dbytes / (dms * 1e-3) / copy_rate}
    with torch.cuda.stream(stream):
        # one GPU's share under expert parallelism, on the same weights; its rows come
        # from the layer's own routing, so the layer runs once first
        layer.forward(x, bufs, stream)
        extra["ep_share"] = ep_share(weights, x, bufs, shape, stream, torch)
        ms, gu_ms, dn_ms, _ = timed_steps(layer, x, bufs, args.steps, args.warmup, stream, torch,
                                          min_warm_ms=HEADLINE_MIN_WARM_MS)
    warm_ms = timed_steps.warm_ms
    R = int(bufs.offsets[-1].item())
    flops_gu = 4.0 * R * shape.d * shape.F
    flops_dn = 2.0 * R * shape.F * shape.d
    achieved = flops_gu / (gu_ms * 1e-3)
    result = {
        "metric": "MoE-layer tokens/s (Qwen3-30B-A3B shape, bf16); grouped-GEMM % of MFMA peak",
        "value": shape.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{shape.name}: T={shape.T} d={shape.d} E={shape.E} top-{shape.k} "
                               f"SwiGLU F={shape.F}, softmax over all then renormalized, dropless, seed 0",
                   "global_batch": shape.T, "parallelism": "single GPU"},
        "warmup_ms": warm_ms,
        "roofline": {"kernel": "grouped gate/up GEMM (+SiLU*up)", "bound": "mfma", "achieved": achieved / 1e12,
                     "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_FLOPS,
                     "traffic": recorded_traffic(), "launch_ms": gu_ms},
        "grouped_gemm": {"ms": gu_ms + dn_ms, "tflops": (flops_gu + flops_dn) / ((gu_ms + dn_ms) * 1e-3) / 1e12,
                         "frac_of_mfma_peak": (flops_gu + flops_dn) / ((gu_ms + dn_ms) * 1e-3) / PEAK_BF16_FLOPS,
                         "down_ms": dn_ms},
    }
    clocks = recorded_clocks()
    if clocks is not None:
        # the MFMA peak at the clock the part sustains under this launch (from the counters)
        peak_gu = PEAK_BF16_FLOPS * clocks[0] / PEAK_CLOCK_GHZ
        peak_dn = PEAK_BF16_FLOPS * clocks[1] / PEAK_CLOCK_GHZ
        result["roofline"]["clock_ghz"] = clocks[0]
        result["roofline"]["frac_at_clock"] = achieved / peak_gu
        result["grouped_gemm"]["down_clock_ghz"] = clocks[1]
        result["grouped_gemm"]["down_frac_at_clock"] = flops_dn / (dn_ms * 1e-3) / peak_dn
    result.update(extra)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
