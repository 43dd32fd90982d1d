"""Benchmark of the multi-tenant LoRA low-precision linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

A step is one pass of the whole hot path over one batch: the Llama-8B-shaped
decoder layer's four projections (qkv, o, gate_up, down) at M = 1 token with
one rank-64 tenant, each through the fused decode path (per-token FP8
quantization, shrink, FP8 GEMM with the adapter epilogue, in one launch per
projection).  Inputs are resident in HBM; the steps are replayed from a HIP
graph, and 4 copies of the weights and adapters are cycled so that no step
finds its 218 MB of weights in the 256 MB Infinity Cache (the method's
kernel timings flush the L2 between runs).  `value` is microseconds per
layer (lower is better).

Also reported: the same layer without an adapter (base-only FP8 GEMM, same
kernel), the unfused paths, per-projection times, the 2048-token prefill
GEMMs (gate_up and down, FP8 and 4-bit weights, 16 and 32 tenant segments)
in TFLOP/s, the roofline of the dominant kernel, and the CPU oracle timed
on a bounded sample of the same layer.
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fp4_gemm_amd as ep  # noqa: E402
from workloads import config  # noqa: E402

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
ROTATE = 4
DEV = "cuda"

METRIC = "µs/layer + %HBM peak at M=1 r=64; FP8 TFLOP/s at M=2048, 32 tenants"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


class Proj:
    """One projection on the device: ROTATE copies of weights and adapters."""

    def __init__(self, g, wfmt="fp8", copies=ROTATE):
        lay = g.layer
        self.g, self.M, self.K, self.N, self.r = g, g.M, g.K, g.N, lay.r
        self.wfmt = wfmt
        self.x = dev(g.x())
        w = dev(g.w())
        if wfmt == "fp8":
            wq = torch.empty(self.N, self.K, dtype=torch.uint8, device=DEV)
            sw = torch.empty(self.N, dtype=torch.float32, device=DEV)
            ep.epilora_quant_weight_fp8(w, wq, sw)
            self.w = [(wq, dict(sw=sw))] + [(wq.clone(), dict(sw=sw.clone())) for _ in range(copies - 1)]
        else:
            wc = torch.empty(self.N, self.K // 2, dtype=torch.uint8, device=DEV)
            bs = torch.empty(self.N, self.K // 16, dtype=torch.uint8, device=DEV)
            gs = torch.empty(1, dtype=torch.float32, device=DEV)
            ws = ep.new_workspace(ep.OP_QUANT_W4, 1, self.N, self.K, 16)
            ep.epilora_quant_weight_fp4(w, wc, bs, gs, ws)
            self.w = [(wc, dict(bs=bs, gs=gs))] + [(wc.clone(), dict(bs=bs.clone(), gs=gs.clone()))
                                                   for _ in range(copies - 1)]
        del w
        A, B = dev(g.A()), dev(g.B())
        self.A = [A] + [A.clone() for _ in range(copies - 1)]
        self.B = [B] + [B.clone() for _ in range(copies - 1)]
        self.idx = dev(lay.idx.astype(np.int32))
        self.mask = None if lay.mask is None else dev(lay.mask.astype(np.uint8))
        self.ranks = None if lay.ranks is None else dev(lay.ranks.astype(np.int32))
        self.scale = lay.scale
        self.y = torch.empty(self.M, self.N, dtype=torch.bfloat16, device=DEV)
        self.xq = torch.empty(self.M, self.K, dtype=torch.uint8, device=DEV)
        self.sx = torch.empty(self.M, dtype=torch.float32, device=DEV)
        self.z = torch.empty(self.M, self.r, dtype=torch.float32, device=DEV)
        self.ws_dec = ep.new_workspace(ep.OP_DECODE, self.M, self.N, self.K, self.r)
        self.ws_shr = ep.new_workspace(ep.OP_SHRINK, self.M, self.N, self.K, self.r)
        self.copies = copies

    def with_batch(self, g):
        """The same projection (the same device weights and adapters) for the
        batch of another layer of the same shapes."""
        q = Proj.__new__(Proj)
        q.__dict__.update(self.__dict__)
        lay = g.layer
        q.g, q.M = g, g.M
        q.x = dev(g.x())
        q.idx = dev(lay.idx.astype(np.int32))
        q.mask = None if lay.mask is None else dev(lay.mask.astype(np.uint8))
        q.ranks = None if lay.ranks is None else dev(lay.ranks.astype(np.int32))
        q.y = torch.empty(q.M, q.N, dtype=torch.bfloat16, device=DEV)
        q.xq = torch.empty(q.M, q.K, dtype=torch.uint8, device=DEV)
        q.sx = torch.empty(q.M, dtype=torch.float32, device=DEV)
        q.z = torch.empty(q.M, q.r, dtype=torch.float32, device=DEV)
        q.ws_dec = ep.new_workspace(ep.OP_DECODE, q.M, q.N, q.K, q.r)
        q.ws_shr = ep.new_workspace(ep.OP_SHRINK, q.M, q.N, q.K, q.r)
        return q

    def adapters(self, c):
        c %= self.copies
        return dict(B=self.B[c], idx=self.idx, ranks=self.ranks, mask=self.mask, scale=self.scale)

    # paths ------------------------------------------------------------------
    def fused(self, c):
        w, kw = self.w[c % self.copies]
        ep.epilora_decode_lora(self.x, w, self.y, A=self.A[c % self.copies], ws=self.ws_dec, xq_out=self.xq,
                               sx_out=self.sx, **self.adapters(c), **kw)

    def fused_base(self, c):
        w, kw = self.w[c % self.copies]
        ep.epilora_decode_lora(self.x, w, self.y, ws=self.ws_dec, xq_out=self.xq, sx_out=self.sx, **kw)

    def quant(self, c):
        ep.epilora_quant_act(self.x, self.xq, self.sx)

    def shrink(self, c):
        ep.epilora_lora_shrink(self.x, self.A[c % self.copies], self.idx, self.z, self.ws_shr, ranks=self.ranks,
                               mask=self.mask)

    def gemm_lora(self, c):
        w, kw = self.w[c % self.copies]
        ep.epilora_gemm_lora(self.xq, self.sx, w, self.y, z=self.z, ws=self.ws_shr, **self.adapters(c), **kw)

    def gemm_base(self, c):
        w, kw = self.w[c % self.copies]
        ep.epilora_gemm_lora(self.xq, self.sx, w, self.y, **kw)

    def expand(self, c):
        ep.epilora_lora_expand_add(self.z, self.B[c % self.copies], self.idx, self.scale, self.y, self.ws_shr,
                                   ranks=self.ranks, mask=self.mask)

    # algorithmic counts -------------------------------------------------------
    def adapter_ranks(self):
        lay = self.g.layer
        act = [int(a) for a, m in zip(lay.idx, lay.mask if lay.mask is not None else [1] * self.M)
               if 0 <= a < lay.L and m]
        distinct = sorted(set(act))
        rk = lambda a: lay.r if lay.ranks is None else int(lay.ranks[a])
        return act, distinct, rk

    def bytes(self):
        act, distinct, rk = self.adapter_ranks()
        if self.wfmt == "fp8":
            wb = self.K * self.N + 4 * self.N
        else:
            wb = self.K * self.N // 2 + self.K * self.N // 16 + 4
        ab = sum(2 * rk(a) * (self.K + self.N) for a in distinct)
        return wb + ab + 2 * self.M * self.K + 2 * self.M * self.N

    def flops(self):
        act, _, rk = self.adapter_ranks()
        return 2 * self.M * self.N * self.K + sum(2 * rk(a) * (self.K + self.N) for a in act)


def graph_of(fns, copies, only=None):
    """Capture `copies` rounds of fns (round c uses weight copy c) in one graph,
    or only round `only`."""
    rounds = range(copies) if only is None else [only]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in rounds:  # warm (first-launch costs out of the capture)
            for f in fns:
                f(c)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in rounds:
            for f in fns:
                f(c)
    torch.cuda.synchronize()
    return g


def time_graph(g, rounds, warmup):
    """Milliseconds per replay of g: events on the replay stream."""
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(rounds):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / rounds


def per_step_us(projs, fn_names, steps, warmup):
    """Microseconds per step (a step = fn_names over projs, on one weight
    copy): `warmup` untimed steps, then exactly `steps` timed ones between
    two synchronizations, timed with events on the stream the graphs replay
    on.  Steps run from one graph that holds a step on each weight copy in
    turn; a remainder of steps % copies runs from one-step graphs."""
    fns = [getattr(p, n) for p in projs for n in fn_names]
    full = graph_of(fns, ROTATE)
    single = [graph_of(fns, ROTATE, only=c) for c in range(ROTATE)]

    def run(n):
        for _ in range(n // ROTATE):
            full.replay()
        for c in range(n % ROTATE):
            single[c].replay()

    run(warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run(steps)
    e1.record()
    torch.cuda.synchronize()
    return 1000.0 * e0.elapsed_time(e1) / steps, steps


def per_call_us(projs, fn_names, steps, warmup):
    """Microseconds per pass of fn_names over projs for the diagnostic
    figures: one graph holds a pass over each weight copy, so that short
    kernels are not paced by graph launches."""
    fns = [getattr(p, n) for p in projs for n in fn_names]
    g = graph_of(fns, ROTATE)
    rounds = max(1, steps // ROTATE)
    ms = time_graph(g, rounds, max(1, warmup // ROTATE))
    return 1000.0 * ms / ROTATE


def decode_72b(steps, warmup):
    """The 72B-shaped PreFT decode layer (qkv 8192->10240, o 8192->8192,
    gate_up 8192->59136, down 29568->8192; 512 rank-16 adapters, Zipf(1.1)
    tenants, the first ceil(0.75 M) tokens adapted) through the fused path at
    M = 1, 8 and 64: microseconds per layer and the fraction of HBM peak over
    the layer's algorithmic bytes.  One copy of the weights (878 MB per layer,
    more than the 256 MB Infinity Cache) serves every batch."""
    out = {}
    base = None
    for M in (1, 8, 64):
        layer = config(4, M=M)
        log(f"72B decode layer M={M} ...")
        if base is None:
            base = [Proj(g, copies=1) for g in layer.gemms]
            projs = base
        else:
            projs = [p.with_batch(g) for p, g in zip(base, layer.gemms)]
        torch.cuda.synchronize()
        us, _ = per_step_us(projs, ["fused"], steps, warmup)
        nbytes = sum(p.bytes() for p in projs)
        out[f"M{M}"] = {"fused_us": round(us, 2), "bytes": nbytes, "GBps": round(nbytes / us / 1e3, 1),
                        "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                        "adapted_tokens": int((layer.mask != 0).sum()),
                        "distinct_tenants": len(projs[0].adapter_ranks()[1])}
        if projs is not base:
            del projs
    del base
    torch.cuda.empty_cache()
    return out


def cpu_baseline(layer, frac=4, min_seconds=10.0, max_reps=1000):
    """The oracle on a bounded sample of the decode layer: every frac-th
    output channel of each projection (its weights quantized by the oracle
    outside the timed region), repeated until about min_seconds of CPU work
    have been timed; the mean time of one pass, scaled by frac, is reported
    in microseconds per layer."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    cases = []
    for g in layer.gemms:
        cols = np.arange(0, g.N, frac)
        wq, sw = oracle.quant_weight_fp8(g.w()[cols])
        cases.append((g.x(), g.A(), g.B()[:, cols], wq, sw))
    timed, reps = 0.0, 0
    while reps < max_reps and (timed < min_seconds or reps < 2):
        t0 = time.perf_counter()
        for x, A, B, wq, sw in cases:
            oracle.linear_lora(x, A, B, layer.idx, layer.scale, wq=wq, sw=sw, ranks=layer.ranks, mask=layer.mask)
        timed += time.perf_counter() - t0
        reps += 1
    us = timed / reps * frac * 1e6
    return {"value": round(us, 1), "unit": "us/layer", "cores": int(threads), "kind": "oracle",
            "sample": f"Llama-8B decode layer (M=1, r=64): every {frac}th output channel of each of the 4 "
                      f"projections (fp64 oracle incl. the FP8 decode of those weights), {reps} passes, "
                      f"{timed:.1f} s timed, scaled x{frac}; host has {os.cpu_count()} cpus"}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_gate_up_traffic.txt")
CSRC = os.path.join(ROOT, "fp4_gemm_amd", "csrc")


def kernel_source_digest():
    """sha256 over the kernel sources, to tell whether recorded counters are
    still those of the kernel that runs."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".h", ".hip")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary, or None when there is none or the kernel
    sources have changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        if kv.get("kernel_source_sha256") != kernel_source_digest():
            return None
        return int(float(kv["traffic_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def traffic_probe(args):
    """Dispatches for the HBM counters (run under rocprofv3 --pmc): a plain
    copy of 1 GiB (the calibration kernel of known size), then the fused
    gate_up projection over its rotated copies, eagerly (one dispatch per
    call, no graph)."""
    torch.cuda.set_device(0)
    ep.lib()
    src = torch.empty(1 << 30, dtype=torch.uint8, device=DEV).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    layer = config(2)
    p = Proj([g for g in layer.gemms if g.name == "gate_up"][0])
    for i in range(args.steps):
        p.fused(i % ROTATE)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "traffic", "copy_bytes": 1 << 30, "gate_up_launches": args.steps,
                      "algorithmic_bytes_per_launch": p.bytes()}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-72b", action="store_true", help="skip the 72B-shaped decode layer")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only the dispatches the HBM-counter runs measure (see traffic_probe)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer shards by tensor parallelism, which is "
              "not part of this build; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.traffic_probe:
        traffic_probe(args)
        return
    torch.cuda.set_device(0)
    ep.lib()

    # ---- headline: the Llama-8B decode layer, M = 1, one rank-64 tenant ----
    layer = config(2)
    log("setting up the decode layer ...")
    projs = [Proj(g) for g in layer.gemms]
    torch.cuda.synchronize()
    fused_us, timed_steps = per_step_us(projs, ["fused"], args.steps, args.warmup)
    base_us, _ = per_step_us(projs, ["fused_base"], args.steps, args.warmup)
    serial_us = per_call_us(projs, ["quant", "shrink", "gemm_lora"], args.steps, args.warmup)
    separate_us = per_call_us(projs, ["quant", "gemm_base", "shrink", "expand"], args.steps, args.warmup)
    gemm_only_us = per_call_us(projs, ["gemm_base"], args.steps, args.warmup)
    per_proj = {}
    for p in projs:
        f_us = per_call_us([p], ["fused"], args.steps, args.warmup)
        b_us = per_call_us([p], ["fused_base"], args.steps, args.warmup)
        per_proj[p.g.name] = {"fused_us": round(f_us, 2), "base_us": round(b_us, 2),
                              "bytes": p.bytes(), "GBps": round(p.bytes() / f_us / 1e3, 1)}
    layer_bytes = sum(p.bytes() for p in projs)
    dom = max(projs, key=lambda p: p.bytes())  # gate_up: the dominant kernel
    dom_us = per_proj[dom.g.name]["fused_us"]
    dom_gbs = dom.bytes() / dom_us / 1e3
    log(f"decode layer: fused {fused_us:.1f} us, base {base_us:.1f} us")

    # ---- prefill: M = 2048, tenant segments ----
    prefill = {}
    if not args.no_prefill:
        for wfmt, segs in (("fp8", 32), ("fp8", 16), ("fp4", 16)):
            lay5 = config(5, segments=segs, wfmt=wfmt)
            for g in lay5.gemms:
                log(f"prefill {wfmt} {segs} segments {g.name} ...")
                p = Proj(g, wfmt, copies=3)
                p.quant(0)
                p.shrink(0)
                gemm_ms = time_graph(graph_of([p.gemm_lora], 3), 10, 2) / 3
                path_ms = time_graph(graph_of([p.quant, p.shrink, p.gemm_lora], 3), 5, 1) / 3
                prefill[f"{g.name}_{wfmt}_{segs}seg"] = {
                    "gemm_us": round(gemm_ms * 1e3, 1), "path_us": round(path_ms * 1e3, 1),
                    "gemm_tflops": round(p.flops() / gemm_ms / 1e9, 1),
                    "path_tflops": round(p.flops() / path_ms / 1e9, 1),
                    "gemm_frac_fp8_peak": round(p.flops() / gemm_ms / 1e9 / FP8_PEAK_TFLOPS, 4)}
                del p
                torch.cuda.empty_cache()

    d72 = None
    if not args.no_72b:
        d72 = decode_72b(max(20, args.steps // 4), max(4, args.warmup // 4))

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle on a sample ...")
        cpu = cpu_baseline(layer)

    out = {
        "metric": METRIC,
        "value": round(fused_us, 2),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": timed_steps,
        "warmup": args.warmup,
        "ms_per_step": round(fused_us / 1000.0, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 (fp32 accumulate)",
        "data": "synthetic (seeded; Llama-8B layer shapes, random adapters)",
        "config": {"workload": "Llama-8B-shaped decode layer (qkv 4096->6144, o 4096->4096, "
                               "gate_up 4096->28672, down 14336->4096), M=1 token, one rank-64 tenant, "
                               "FP8 e4m3 per-channel weights, fused decode path, HIP graph replay, "
                               f"{ROTATE} rotated weight copies",
                   "M": 1, "rank": 64, "tenants": 1},
        "hbm_frac": round(layer_bytes / fused_us / 1e3 / HBM_PEAK_GBS, 4),
        "layer_bytes": layer_bytes,
        "base_only_us": round(base_us, 2),
        "fused_over_base": round(fused_us / base_us, 3),
        "gemm_only_us": round(gemm_only_us, 2),
        "serialized_us": round(serial_us, 2),
        "separate_kernels_us": round(separate_us, 2),
        "per_projection": per_proj,
        "roofline": {"kernel": f"decode_kernel ({dom.g.name}, fused)", "bound": "hbm",
                     "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(),
                     "algorithmic_bytes": dom.bytes(), "launch_us": dom_us},
        "prefill": prefill,
        "decode_72b_preft": d72,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
