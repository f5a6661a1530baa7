"""Benchmark: one MoE layer, forward + backward, on one MI355X.

A step is one pass of the whole layer -- routing/layout, dispatch, expert FFN
(grouped GEMMs with fused SwiGLU), combine, and the full backward -- over one
batch of seeded synthetic inputs already resident in HBM.  Prints ONE JSON
line.  The default workload is the Kimi-shaped expert share: 2048 tokens x
top-8 = 16,384 routed rows, hidden 7168, 6 local experts of intermediate 2048,
Zipf(s=1.0) expert loads, bf16.

Both schedules of the layer are timed: the staged one (one kernel per step
over all rows) and the minibatch-pipelined one (communication and GEMM
streams); `value` is the throughput of --schedule (default: pipelined).  The
per-stage times, MFMA and HBM fractions and the roofline come from a staged
pass with HIP events around every kernel on the layer's stream.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--schedule staged|pipelined] [--minibatch-rows N]
                    [--comm-cus N] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA (the MX-scaled fp8 instruction)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

# GEMM stages whose operands are MXFP8 when the layer runs in MXFP8 (the
# weight gradients stay bf16)
MX_GEMMS = ("gemm_gate_up_swiglu", "gemm_down", "gemm_dgrad_down_swiglu_bwd",
            "gemm_dgrad_gate_up")
CSRC = os.path.join(ROOT, "mixture_experts_layer_offsets_amd", "csrc")
KERNEL_SOURCES = {
    "gemm_nt_kernel<2>": ("gemm.hip", "gemm_common.h", "row_tile.h", "tile_epilogue.h"),
    "gemm_mx_kernel<2>": ("gemm_mx.hip", "gemm_common.h", "mx_device.h", "row_tile.h",
                          "tile_epilogue.h"),
}

FWD_STAGES = ["route+layout", "dispatch", "gemm_gate_up_swiglu", "gemm_down", "shared",
              "combine"]
BWD_STAGES = ["reverse_combine", "gemm_dgrad_down_swiglu_bwd", "gemm_wgrad_down",
              "gemm_dgrad_gate_up", "gemm_wgrad_gate_up", "shared_bwd",
              "router_bwd+reverse_dispatch"]


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="kimi-bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=2048,
                    help="tokens of the bounded oracle sample (CPU baseline)")
    ap.add_argument("--schedule", choices=("staged", "pipelined"), default="pipelined",
                    help="schedule whose throughput is `value` (both are timed and reported)")
    ap.add_argument("--minibatch-rows", type=int, default=0,
                    help="pipelined schedule: routed rows per minibatch (0 = library default)")
    ap.add_argument("--ring-slots", type=int, default=0,
                    help="pipelined schedule: minibatches dispatched ahead of the gate/up GEMM "
                         "(0 = library default)")
    ap.add_argument("--comm-cus", type=int, default=0,
                    help="pipelined schedule: CUs of the communication stream (0 = share all)")
    ap.add_argument("--sweep-minibatch", default="",
                    help="comma-separated minibatch sizes (routed rows): also time the pipelined "
                         "schedule at each and report forward/backward ms per size")
    ap.add_argument("--decode-tokens", type=int, default=0,
                    help="also time the few-token inference forward (moe_decode_fwd) on the first "
                         "N tokens of the workload, against moe_layer_fwd on the same tokens")
    ap.add_argument("--mx-wgrad", action="store_true",
                    help="MXFP8 workloads: weight-gradient GEMMs on MX operands too")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates HBM byte counters)")
    return ap.parse_args()


def copy_probe():
    """A plain device-to-device copy of known size: what FETCH_SIZE/WRITE_SIZE
    read for it calibrates the counters used for the layer's kernels."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_per_launch": n}), flush=True)


def _algorithmic(w):
    """Algorithmic flops / bytes of the layer's stages (per step)."""
    R, T, H, I, k = w.T * w.k, w.T, w.H, w.I, w.k
    f = {
        "gemm_gate_up_swiglu": 4.0 * R * H * I,
        "gemm_down": 2.0 * R * H * I,
        "gemm_dgrad_down_swiglu_bwd": 2.0 * R * H * I,
        "gemm_wgrad_down": 2.0 * R * H * I,
        "gemm_dgrad_gate_up": 4.0 * R * H * I,
        "gemm_wgrad_gate_up": 4.0 * R * H * I,
    }
    # bytes per element of a dispatched row: bf16, or an E4M3 code plus a
    # 1/32 share of an E8M0 scale
    xb = 1.0 + 1.0 / 32 if w.mx else 2.0
    b = {
        # unique token rows read once, routed rows written once, + indices
        "dispatch": T * H * 2 + R * H * xb + R * 4,
        # routed rows read once, token rows written once, + weights/indices
        "combine": R * H * 2 + T * H * 2 + R * 8,
        # dOut read once, Y read for dw, dY written, + weights/indices/dw
        "reverse_combine": T * H * 2 + 2 * R * H * 2 + R * 12,
    }
    if w.routing == "supplied":
        # without a router this stage is reverse-dispatch alone: the rows'
        # gradients read once, token rows written once, + indices
        b["router_bwd+reverse_dispatch"] = R * H * 2 + T * H * 2 + R * 4
    return f, b


def sources_sha256(kernel: str) -> str:
    """Hash of the source files a kernel is built from."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def _traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on this workload and the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        ent = json.load(open(path)).get(f"{kernel} {workload}")
        if not ent or ent.get("sources_sha256") != sources_sha256(kernel):
            return None
        return ent["bytes_per_launch"]
    except Exception:
        return None


def cpu_baseline(w, inp, tokens: int):
    """The oracle, as it is, on a bounded sample: the first `tokens` tokens of
    the same workload (same weights and routing), forward + backward."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    sub = dict(inp)
    for key in ("x", "dout", "topk_idx", "topk_w"):
        if sub.get(key) is not None:
            sub[key] = np.ascontiguousarray(inp[key][:tokens])
    t0 = time.perf_counter()
    fw = oracle.forward(sub, w.k, mx=w.mx)
    oracle.backward(sub, fw)
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {tokens} of {w.T} tokens ({tokens * w.k} routed rows) of the "
                      f"same workload, fp64 numpy oracle, forward+backward, {dt:.1f} s"}


def main():
    a = _args()
    if a.copy_probe:
        copy_probe()
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {a.gpus}).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    from mixture_experts_layer_offsets_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from mixture_experts_layer_offsets_amd import build
        build.build(verbose=False)
    import mixture_experts_layer_offsets_amd as m

    w = synth.workload(a.workload)
    inp = synth.make_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def d(x):
        if x is None:
            return None
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            x = x.view(np.int16)
        return torch.from_numpy(x).to(dev)

    shape = m.Shape(w.T, w.H, w.E, w.k, w.I, w.shared_I, m.MOE_MXFP8 if w.mx else m.MOE_BF16)
    layer = m.MoeLayer(shape, dev)
    layer.prepare(d(inp["w_gate"]), d(inp["w_up"]), d(inp["w_down"]), d(inp["ws_gate"]),
                  d(inp["ws_up"]), d(inp["ws_down"]))
    x, wr, bias = d(inp["x"]), d(inp["w_router"]), d(inp["bias"])
    idx, tw, dout = d(inp["topk_idx"]), d(inp["topk_w"]), d(inp["dout"])
    out = torch.empty((w.T, w.H), dtype=torch.int16, device=dev)
    grads = layer.grad_buffers(router=wr is not None)

    n_f, n_b = len(FWD_STAGES) + 1, len(BWD_STAGES) + 1

    def make_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record()
        return evs

    def sched_for(evs):
        """Stage events (None: that boundary is not recorded)."""
        import ctypes
        arr = (ctypes.c_void_p * len(evs))(*[e.cuda_event if e is not None else None
                                              for e in evs])
        s = m.MoeSched()
        s.stage_events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
        s.n_stage_events = len(evs)
        return s, arr

    def step(sf=None, sb=None):
        if a.mx_wgrad and w.mx:
            if sb is None:
                sb = m.MoeSched()
            sb.mx_wgrad = 1
        layer.forward(x, w_router=wr, bias=bias, topk_idx=idx, topk_w=tw, out=out, sched=sf)
        if w.backward:
            layer.backward(dout, x, w_router=wr, grads=grads, sched=sb)

    def pipelined():
        s = m.MoeSched()
        s.schedule = m.MOE_SCHED_PIPELINED
        s.minibatch_rows = a.minibatch_rows
        s.comm_cus = a.comm_cus
        s.ring_slots = a.ring_slots
        return s

    def timed_loop(sf=None, sb=None):
        """K steps of one schedule, no stage events: seconds of wall clock."""
        for _ in range(a.warmup):
            step(sf, sb)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(a.steps):
            step(sf, sb)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    # the timed steps of each schedule
    sp = pipelined()
    wall = {"staged": timed_loop(), "pipelined": timed_loop(sp, sp)}
    elapsed = wall[a.schedule]
    ms = elapsed / a.steps * 1e3

    # per-stage times (staged schedule, HIP events on the layer's stream)
    for _ in range(a.warmup):
        step()
    ev = [(make_events(n_f), make_events(n_b)) for _ in range(a.steps)]
    scheds = [(sched_for(f), sched_for(b)) for f, b in ev]
    torch.cuda.synchronize()
    for (sf, _), (sb, _) in scheds:
        step(sf, sb)
    torch.cuda.synchronize()
    # forward / backward split of the pipelined schedule (events at its joins)
    pev = [(make_events(n_f), make_events(n_b)) for _ in range(a.steps)]
    psched = []
    for f, b in pev:
        (pf, af), (pb, ab) = sched_for(f), sched_for(b)
        for q in (pf, pb):
            q.schedule = m.MOE_SCHED_PIPELINED
            q.minibatch_rows = a.minibatch_rows
            q.comm_cus = a.comm_cus
            q.ring_slots = a.ring_slots
        psched.append(((pf, af), (pb, ab)))
    torch.cuda.synchronize()
    for (pf, _), (pb, _) in psched:
        step(pf, pb)
    torch.cuda.synchronize()
    pipe_fwd = float(np.mean([f[0].elapsed_time(f[-1]) for f, _ in pev]))
    pipe_bwd = float(np.mean([b[0].elapsed_time(b[-1]) for _, b in pev])) if w.backward else None

    def pipelined_split(mb):
        """Forward and backward ms of the pipelined schedule at minibatch mb
        (events at the start and at the join of each direction)."""
        evs = [(make_events(2), make_events(2)) for _ in range(a.steps)]
        run = []
        for f, b in evs:
            (pf, af), (pb, ab) = sched_for([f[0]] + [None] * 5 + [f[1]]), \
                sched_for([b[0]] + [None] * 6 + [b[1]])
            for q in (pf, pb):
                q.schedule = m.MOE_SCHED_PIPELINED
                q.minibatch_rows = mb
                q.comm_cus = a.comm_cus
            run.append(((pf, af), (pb, ab)))
        q = pipelined()
        q.minibatch_rows = mb
        for _ in range(a.warmup):
            step(q, q)
        torch.cuda.synchronize()
        for (pf, _), (pb, _) in run:
            step(pf, pb)
        torch.cuda.synchronize()
        fwd = float(np.mean([f[0].elapsed_time(f[1]) for f, _ in evs]))
        bwd = float(np.mean([b[0].elapsed_time(b[1]) for _, b in evs])) if w.backward else None
        return {"minibatch_rows": mb, "minibatches": -(-w.T * w.k // mb),
                "layer_fwd_ms": fwd, "layer_bwd_ms": bwd}

    sweep = [pipelined_split(int(v)) for v in a.sweep_minibatch.split(",") if v.strip()]

    def decode_bench(n):
        """moe_decode_fwd on the first n tokens (same weights and routing),
        HIP events on the current stream around K calls; bytes = the weights
        of the experts those tokens select (+ the shared expert), read once."""
        sh = m.Shape(n, w.H, w.E, w.k, w.I, w.shared_I, m.MOE_BF16)
        L = m.MoeLayer(sh, dev)
        L.prepare(d(inp["w_gate"]), d(inp["w_up"]), d(inp["w_down"]), d(inp["ws_gate"]),
                  d(inp["ws_up"]), d(inp["ws_down"]))
        kw = dict(w_router=wr, bias=bias)
        if wr is None:
            kw = dict(topk_idx=idx[:n].contiguous(), topk_w=tw[:n].contiguous())
        xs = x[:n].contiguous()

        def timed(fn):
            for _ in range(a.warmup):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(a.steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / a.steps

        t_dec = timed(lambda: L.decode(xs, **kw))
        t_fwd = timed(lambda: L.forward(xs, **kw))
        if wr is None:
            used = len(np.unique(inp["topk_idx"][:n]))
        else:
            used = len(np.unique(L.saved_tensor("topk_idx", torch.int32, (n, w.k)).cpu().numpy()))
        wbytes = (used * 3 * w.H * w.I + 3 * w.H * w.shared_I) * 2
        gbs = wbytes / (t_dec * 1e-3) / 1e9
        return {"tokens": n, "decode_ms": t_dec, "layer_fwd_ms": t_fwd, "experts_read": used,
                "weight_bytes": wbytes, "achieved_GBs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS}

    decode = decode_bench(a.decode_tokens) if a.decode_tokens > 0 and not w.mx else None

    stage_ms = {}
    for i, name in enumerate(FWD_STAGES):
        stage_ms[name] = float(np.mean([f[i].elapsed_time(f[i + 1]) for f, _ in ev]))
    if w.backward:
        for i, name in enumerate(BWD_STAGES):
            stage_ms[name] = float(np.mean([b[i].elapsed_time(b[i + 1]) for _, b in ev]))
    flops, byts = _algorithmic(w)

    def peak(stage):
        mx_stage = stage in MX_GEMMS or (a.mx_wgrad and stage.startswith("gemm_wgrad"))
        return PEAK_FP8_TFLOPS if w.mx and mx_stage else PEAK_BF16_TFLOPS
    mfma = {k: flops[k] / (stage_ms[k] * 1e-3) / 1e12 / peak(k)
            for k in flops if k in stage_ms and stage_ms[k] > 0}
    hbm = {k: byts[k] / (stage_ms[k] * 1e-3) / 1e9 / PEAK_HBM_GBS
           for k in byts if k in stage_ms and stage_ms[k] > 0}

    dom = "gemm_gate_up_swiglu"
    achieved = flops[dom] / (stage_ms[dom] * 1e-3) / 1e12
    kernel = "gemm_mx_kernel<2>" if w.mx else "gemm_nt_kernel<2>"
    traffic = _traffic(kernel, w.name)
    tokens_per_step = w.T
    res = {
        # value is the tokens/s; the grouped-GEMM MFMA and permute HBM
        # fractions are the roofline, mfma_frac and hbm_frac fields
        "metric": "MoE layer fwd+bwd tokens/s on 1 MI355X; grouped-GEMM MFMA % and permute HBM %"
                  if w.backward
                  else "MoE layer fwd tokens/s on 1 MI355X",
        "value": tokens_per_step * a.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("mxfp8 (weight gradients too)" if a.mx_wgrad else "mxfp8") if w.mx else "bf16",
        "data": "synthetic (seeded; random-init weights; supplied Zipf routing)"
                if w.routing == "supplied" else "synthetic (seeded; random-init weights)",
        "config": {"workload": f"{w.name}: T={w.T} tokens, top-{w.k} ({w.T * w.k} routed rows), "
                               f"hidden {w.H}, {w.E} experts of intermediate {w.I}"
                               + (f", shared expert {w.shared_I}" if w.shared_I else "")
                               + (f", Zipf s={w.zipf_s}" if w.routing == "supplied" else ""),
                   "tokens": w.T, "hidden": w.H, "experts": w.E, "top_k": w.k,
                   "inter": w.I, "routed_rows": w.T * w.k},
        "roofline": {"bound": "mfma", "kernel": f"{kernel} "
                     "(gate/up grouped GEMM + SwiGLU epilogue)",
                     "achieved": achieved, "peak": peak(dom), "unit": "TFLOP/s",
                     "frac": achieved / peak(dom), "traffic": traffic,
                     "avg_launch_ms": stage_ms[dom]},
        "stage_ms": stage_ms,
        "mfma_frac": mfma,
        "hbm_frac": hbm,
        "layer_fwd_ms": sum(stage_ms[n] for n in FWD_STAGES),
        "layer_bwd_ms": sum(stage_ms[n] for n in BWD_STAGES) if w.backward else None,
        "schedule": a.schedule,
        "schedules_ms_per_step": {k: v / a.steps * 1e3 for k, v in wall.items()},
        "pipelined": {"layer_fwd_ms": pipe_fwd, "layer_bwd_ms": pipe_bwd,
                      "minibatch_rows": a.minibatch_rows or "default",
                      "comm_cus": a.comm_cus},
    }
    if sweep:
        res["minibatch_sweep"] = sweep
    if decode:
        res["decode"] = decode
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, inp, min(a.cpu_tokens, w.T))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
