"""Benchmark: one MoE layer, forward + backward, on one MI355X.

A step is one pass of the whole layer -- routing/layout, dispatch, expert FFN
(grouped GEMMs with fused SwiGLU), combine, and the full backward -- over one
batch of seeded synthetic inputs already resident in HBM.  Prints ONE JSON
line.  The default workload is the Kimi-shaped expert share: 2048 tokens x
top-8 = 16,384 routed rows, hidden 7168, 6 local experts of intermediate 2048,
Zipf(s=1.0) expert loads, bf16; the same share in MXFP8 (Zipf s=1.2) is timed
beside it (the "kimi_mx" entry).

Both schedules of the layer are timed: the staged one (one kernel per step
over all rows) and the minibatch-pipelined one (communication and GEMM
streams); `value` is the throughput of --schedule (default: pipelined, with
the library's default minibatch: two full waves of 256 x 256 tiles of each
direction's first GEMM).  The pipelined schedule at 2368-row minibatches (the
Kimi-shaped configuration's stated minibatch) is reported beside it.  The
per-stage times, MFMA fractions and the roofline come from a staged pass with
HIP events around every kernel on the layer's stream; the permute stages'
HBM fractions come from a second staged pass in which 1 GiB of scratch is
written and then read back right before each of those stages (the 256 MB
Infinity Cache then holds none of their inputs, and no dirty lines that the
timed stage would have to write back).  The unflushed staged pass also reads
the GEMM tiles' in-kernel counters (shader cycles against the 100 MHz real-
time counter): "gemm_tiles" gives each GEMM stage's shader clock and the
share of its cycles in the K loop and in the epilogue, and
"mfma_frac_at_measured_clock" its MFMA fraction against the peak scaled to
that clock (the published peaks assume 2.4 GHz; under these GEMMs the chip
runs well below it).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--schedule staged|pipelined] [--minibatch-rows N]
                    [--comm-cus N] [--no-cpu-baseline] [--no-companion]
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
PEAK_CLOCK_MHZ = 2400.0       # the engine clock the MFMA peaks are quoted at

# GEMM stages whose operands are MXFP8 when the layer runs in MXFP8 (the
# weight gradients stay bf16)
MX_GEMMS = ("gemm_gate_up_swiglu", "gemm_down", "gemm_dgrad_down_swiglu_bwd",
            "gemm_dgrad_gate_up")
CSRC = os.path.join(ROOT, "mixture_experts_layer_offsets_amd", "csrc")
KERNEL_SOURCES = {
    "gemm_nt_kernel<2>": ("gemm.hip", "gemm_common.h", "row_tile.h", "tile_epilogue.h",
                          "tile_order.h", "kernels.h", "common.h"),
    "gemm_mx_kernel<2, 0>": ("gemm_mx.hip", "gemm_common.h", "mx_device.h", "row_tile.h",
                             "tile_epilogue.h", "tile_order.h", "kernels.h", "common.h"),
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
    ap.add_argument("--no-companion", action="store_true",
                    help="do not time the companion workload (kimi-mx beside kimi-bf16)")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the flushed pass that times the permute stages")
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
    # bytes per element of a dispatched row: bf16, or an E4M3 code, a 1/32
    # share of an E8M0 scale and the bf16 round trip the weight gradients read
    xb = 1.0 + 1.0 / 32 + 2.0 if w.mx else 2.0
    b = {
        # unique token rows read once, routed rows written once, + indices
        "dispatch": T * H * 2 + R * H * xb + R * 4,
        # routed rows read once, token rows written once, + weights/indices
        "combine": R * H * 2 + T * H * 2 + R * 8,
        # dOut read once, Y read for dw, dY written, + weights/indices/dw;
        # with MXFP8 also dY's codes and scales (the down data gradient's operand)
        "reverse_combine": T * H * 2 + 2 * R * H * 2 + R * 12
        + (R * H * (1.0 + 1.0 / 32) if w.mx else 0.0),
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


def _tile_clocks(st, names, steps) -> dict:
    """Per GEMM stage, from the tiles' in-kernel counters (moe_sched
    kernel_stamps: tiles, shader cycles, prologue + K-loop cycles, epilogue
    cycles, 100 MHz real-time ticks): the shader clock the tiles ran at and
    where their cycles went."""
    out = {}
    for i, name in enumerate(names):
        tiles, cyc, loop, epi, ticks = (int(v) for v in st[i][:5])
        if tiles == 0 or ticks == 0:
            continue
        out[name] = {"clock_mhz": cyc / ticks * 100.0,
                     "tiles_per_step": tiles / steps,
                     "cycles_per_tile": cyc / tiles,
                     "loop_share": loop / cyc,
                     "epilogue_share": epi / cyc}
    return out


def _dtype_name(w, mx_wgrad=False) -> str:
    """The arithmetic the expert GEMMs run in."""
    if not w.mx:
        return "bf16"
    s = "mxfp8" if w.wfmt == "e4m3" else f"mxfp8 activations x {w.wfmt} MX weights"
    return s + " (weight gradients too)" if mx_wgrad else s


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
    cores, blas = os.cpu_count() or 1, "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            cores = max(p.get("num_threads", 1) for p in info)
            blas = ", ".join(f"{p.get('internal_api')} {p.get('version')} "
                             f"({p.get('architecture')})" for p in info)
    except Exception:
        pass
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    sub = dict(inp)
    for key in ("x", "dout", "topk_idx", "topk_w"):
        if sub.get(key) is not None:
            sub[key] = np.ascontiguousarray(inp[key][:tokens])
    t0 = time.perf_counter()
    fw = oracle.forward(sub, w.k, mx=w.mx)
    oracle.backward(sub, fw)
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu, "blas": blas,
            "sample": f"first {tokens} of {w.T} tokens ({tokens * w.k} routed rows) of the "
                      f"same workload, fp64 numpy oracle, forward+backward, {dt:.1f} s"}


def default_minibatch(w, fwd: bool, cus: int = 256) -> int:
    """The library's default minibatch (include/moe.h, moe_sched.minibatch_rows):
    rows for two full waves of 256 x 256 tiles of the direction's first GEMM
    (gate/up forward: 2I columns; down data gradient backward: I columns),
    in the forward at least half the rows, at least max(256, ceil(R/1024)),
    at most R."""
    R = w.T * w.k
    n_tiles = -(-(2 * w.I if fwd else w.I) // 256)
    mb = -(-2 * cus // n_tiles) * 256
    if fwd:
        mb = max(mb, (R + 1) // 2)
    return min(max(mb, 256, -(-R // 1024)), R)


class Bench:
    """One workload's layer, inputs and buffers on the device, and its timings."""

    def __init__(self, a, name):
        import numpy as np
        import torch

        import mixture_experts_layer_offsets_amd as m
        import synth
        self.a, self.m, self.torch, self.np = a, m, torch, np
        self.w = w = synth.workload(name)
        self.inp = inp = synth.make_inputs(w, threads=16)
        dev = self.dev = torch.device("cuda:0")

        def d(x):
            if x is None:
                return None
            x = np.ascontiguousarray(x)
            if x.dtype == np.uint16:
                x = x.view(np.int16)
            return torch.from_numpy(x).to(dev)
        self.d = d
        dtype = {v: k for k, v in m.WEIGHT_FORMAT.items()}[w.wfmt] if w.mx else m.MOE_BF16
        shape = m.Shape(w.T, w.H, w.E, w.k, w.I, w.shared_I, dtype)
        self.layer = m.MoeLayer(shape, dev)
        self.layer.prepare(d(inp["w_gate"]), d(inp["w_up"]), d(inp["w_down"]),
                           d(inp["ws_gate"]), d(inp["ws_up"]), d(inp["ws_down"]))
        self.x, self.wr, self.bias = d(inp["x"]), d(inp["w_router"]), d(inp["bias"])
        self.idx, self.tw, self.dout = d(inp["topk_idx"]), d(inp["topk_w"]), d(inp["dout"])
        self.out = torch.empty((w.T, w.H), dtype=torch.int16, device=dev)
        self.grads = self.layer.grad_buffers(router=self.wr is not None)
        self.n_f, self.n_b = len(FWD_STAGES) + 1, len(BWD_STAGES) + 1
        self._keep = []          # ctypes objects that must outlive their calls

    # -- schedules
    def sched(self, pipelined=False, mb=None, evs=None, hook=None, stamps=None):
        import ctypes
        s = self.m.MoeSched()
        if stamps is not None:
            s.kernel_stamps = stamps.data_ptr()
        if pipelined:
            s.schedule = self.m.MOE_SCHED_PIPELINED
            s.minibatch_rows = self.a.minibatch_rows if mb is None else mb
            s.comm_cus = self.a.comm_cus
            s.ring_slots = self.a.ring_slots
        if evs is not None:
            arr = (ctypes.c_void_p * len(evs))(*[e.cuda_event if e is not None else None
                                                  for e in evs])
            s.stage_events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
            s.n_stage_events = len(evs)
            self._keep.append(arr)
        if hook is not None:
            s.stage_hook = hook
        return s

    def step(self, sf=None, sb=None):
        if self.a.mx_wgrad and self.w.mx:
            if sb is None:
                sb = self.m.MoeSched()
            sb.mx_wgrad = 1
        self.layer.forward(self.x, w_router=self.wr, bias=self.bias, topk_idx=self.idx,
                           topk_w=self.tw, out=self.out, sched=sf)
        if self.w.backward:
            self.layer.backward(self.dout, self.x, w_router=self.wr, grads=self.grads, sched=sb)

    def events(self, n):
        evs = [self.torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record()
        return evs

    # -- timings
    def timed_loop(self, sf=None, sb=None):
        """K steps of one schedule, no stage events: seconds of wall clock."""
        torch = self.torch
        for _ in range(self.a.warmup):
            self.step(sf, sb)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(self.a.steps):
            self.step(sf, sb)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def staged_stages(self, flush=None):
        """Per-stage ms of the staged schedule (HIP events on the layer's
        stream around every stage).  With ``flush`` (a device buffer), the
        buffer is overwritten and read back right before the stages named in
        FLUSH_FWD / FLUSH_BWD."""
        np, torch = self.np, self.torch
        hooks = (None, None)
        if flush is not None:
            def mk(stages):
                def fn(_user, stage):
                    if stage in stages:
                        # write the scratch, then read it back: the write
                        # evicts the Infinity Cache, the read leaves it
                        # holding clean, unrelated lines (a write alone
                        # leaves dirty lines the timed stage would have to
                        # write back)
                        flush.fill_(stage)
                        flush.view(torch.int64).sum()  # a plain read, no widening copy
                return _lib.STAGE_HOOK(fn)
            from mixture_experts_layer_offsets_amd import _lib
            hooks = (mk(FLUSH_FWD), mk(FLUSH_BWD))
            self._keep.extend(hooks)
        for _ in range(self.a.warmup):
            self.step()
        ev = [(self.events(self.n_f), self.events(self.n_b)) for _ in range(self.a.steps)]
        # the unflushed pass also collects the GEMM tiles' in-kernel timing
        stamps = None if flush is not None else tuple(
            torch.zeros((n, 8), dtype=torch.int64, device="cuda") for n in (self.n_f, self.n_b))
        scheds = [(self.sched(evs=f, hook=hooks[0], stamps=stamps and stamps[0]),
                   self.sched(evs=b, hook=hooks[1], stamps=stamps and stamps[1]))
                  for f, b in ev]
        torch.cuda.synchronize()
        for sf, sb in scheds:
            self.step(sf, sb)
        torch.cuda.synchronize()
        if stamps is not None:
            self.clocks = _tile_clocks(stamps[0].cpu().numpy(), FWD_STAGES, self.a.steps)
            if self.w.backward:
                self.clocks.update(_tile_clocks(stamps[1].cpu().numpy(), BWD_STAGES,
                                                self.a.steps))
        ms = {}
        for i, name in enumerate(FWD_STAGES):
            ms[name] = float(np.mean([f[i].elapsed_time(f[i + 1]) for f, _ in ev]))
        if self.w.backward:
            for i, name in enumerate(BWD_STAGES):
                ms[name] = float(np.mean([b[i].elapsed_time(b[i + 1]) for _, b in ev]))
        return ms

    def pipelined_split(self, mb):
        """Forward and backward ms of the pipelined schedule at minibatch mb
        (0 = default; events at the start and at the join of each direction)."""
        np, torch = self.np, self.torch
        evs = [(self.events(2), self.events(2)) for _ in range(self.a.steps)]
        run = [(self.sched(True, mb, [f[0]] + [None] * 5 + [f[1]]),
                self.sched(True, mb, [b[0]] + [None] * 6 + [b[1]])) for f, b in evs]
        q = self.sched(True, mb)
        for _ in range(self.a.warmup):
            self.step(q, q)
        torch.cuda.synchronize()
        for pf, pb in run:
            self.step(pf, pb)
        torch.cuda.synchronize()
        fwd = float(np.mean([f[0].elapsed_time(f[1]) for f, _ in evs]))
        bwd = float(np.mean([b[0].elapsed_time(b[1]) for _, b in evs])) if self.w.backward \
            else None
        w = self.w
        return {"minibatch_rows": mb or "default",
                "minibatches": {"forward": -(-w.R // (mb or default_minibatch(w, True))),
                                "backward": -(-w.R // (mb or default_minibatch(w, False)))},
                "layer_fwd_ms": fwd, "layer_bwd_ms": bwd,
                "tokens_per_s": w.T / ((fwd + (bwd or 0.0)) * 1e-3)}

    def measure(self, flush=None):
        """The whole measurement of this workload (without the CPU baseline)."""
        a, w = self.a, self.w
        sp = self.sched(True)
        wall = {"staged": self.timed_loop(), "pipelined": self.timed_loop(sp, sp)}
        elapsed = wall[a.schedule]
        stage_ms = self.staged_stages()
        flushed = self.staged_stages(flush) if flush is not None else None
        flops, byts = _algorithmic(w)

        def peak(stage):
            mx_stage = stage in MX_GEMMS or (a.mx_wgrad and stage.startswith("gemm_wgrad"))
            return PEAK_FP8_TFLOPS if w.mx and mx_stage else PEAK_BF16_TFLOPS
        mfma = {k: flops[k] / (stage_ms[k] * 1e-3) / 1e12 / peak(k)
                for k in flops if k in stage_ms and stage_ms[k] > 0}
        perm_ms = flushed if flushed is not None else stage_ms
        hbm = {k: byts[k] / (perm_ms[k] * 1e-3) / 1e9 / PEAK_HBM_GBS
               for k in byts if k in perm_ms and perm_ms[k] > 0}
        hbm_cached = {k: byts[k] / (stage_ms[k] * 1e-3) / 1e9 / PEAK_HBM_GBS
                      for k in byts if k in stage_ms and stage_ms[k] > 0}
        dom = "gemm_gate_up_swiglu"
        achieved = flops[dom] / (stage_ms[dom] * 1e-3) / 1e12
        fmt_code = {"e4m3": 0, "e2m3": 2, "e3m2": 3, "e2m1": 4}[w.wfmt]
        kernel = f"gemm_mx_kernel<2, {fmt_code}>" if w.mx else "gemm_nt_kernel<2>"
        res = {
            "value": w.T * a.steps / elapsed,
            "ms_per_step": elapsed / a.steps * 1e3,
            "roofline": {"bound": "mfma", "kernel": f"{kernel} "
                         "(gate/up grouped GEMM + SwiGLU epilogue)",
                         "achieved": achieved, "peak": peak(dom), "unit": "TFLOP/s",
                         "frac": achieved / peak(dom), "traffic": _traffic(kernel, w.name),
                         "avg_launch_ms": stage_ms[dom]},
            "stage_ms": stage_ms,
            "mfma_frac": mfma,
            "hbm_frac": hbm,
            "layer_fwd_ms": sum(stage_ms[n] for n in FWD_STAGES),
            "layer_bwd_ms": sum(stage_ms[n] for n in BWD_STAGES) if w.backward else None,
            "schedules_ms_per_step": {k: v / a.steps * 1e3 for k, v in wall.items()},
        }
        clocks = getattr(self, "clocks", {})
        if clocks:
            res["gemm_tiles"] = clocks
            res["mfma_frac_at_measured_clock"] = {
                k: v * PEAK_CLOCK_MHZ / clocks[k]["clock_mhz"] for k, v in mfma.items()
                if k in clocks and clocks[k]["clock_mhz"] > 0}
        if flushed is not None:
            res["permute_stage_ms_after_flush"] = {k: flushed[k] for k in byts if k in flushed}
            res["hbm_frac_without_flush"] = hbm_cached
        res["pipelined"] = dict(self.pipelined_split(a.minibatch_rows), comm_cus=a.comm_cus)
        if w.name.startswith("kimi"):
            res["pipelined_minibatch_2368"] = self.pipelined_split(2368)
        return res


# Stage boundaries before which the flushed pass overwrites the scratch
# buffer: dispatch and combine (forward), reverse-combine and
# reverse-dispatch (backward).  A flush lands in the interval of the stage
# before (route+layout, shared expert; the shared backward), which that pass
# does not report.
FLUSH_FWD = (FWD_STAGES.index("dispatch"), FWD_STAGES.index("combine"))
FLUSH_BWD = (BWD_STAGES.index("reverse_combine"), BWD_STAGES.index("router_bwd+reverse_dispatch"))


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

    from mixture_experts_layer_offsets_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from mixture_experts_layer_offsets_amd import build
        build.build(verbose=False)
    torch.cuda.set_device(torch.device("cuda:0"))
    flush = None if a.no_flush else torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    b = Bench(a, a.workload)
    w = b.w
    main_res = b.measure(flush)
    sweep = [b.pipelined_split(int(v)) for v in a.sweep_minibatch.split(",") if v.strip()]
    decode = decode_bench(b, a.decode_tokens) if a.decode_tokens > 0 and not w.mx else None
    cpu = None if a.no_cpu_baseline else cpu_baseline(w, b.inp, min(a.cpu_tokens, w.T))
    inp_main = b.inp
    companion = None
    if not a.no_companion and w.name == "kimi-bf16":
        del b
        torch.cuda.empty_cache()
        c = Bench(a, "kimi-mx")
        r = c.measure(flush)
        companion = {"workload": _describe(c.w), "dtype": "mxfp8", **r}
        del c
    res = {
        # value is the tokens/s; the grouped-GEMM MFMA and permute HBM
        # fractions are the roofline, mfma_frac and hbm_frac fields
        "metric": "MoE layer fwd+bwd tokens/s on 1 MI355X; grouped-GEMM MFMA % and permute HBM %"
                  if w.backward
                  else "MoE layer fwd tokens/s on 1 MI355X",
        "value": main_res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": _dtype_name(w, a.mx_wgrad),
        "data": "synthetic (seeded; random-init weights; supplied Zipf routing)"
                if w.routing == "supplied" else "synthetic (seeded; random-init weights)",
        "config": {"workload": _describe(w),
                   "tokens": w.T, "hidden": w.H, "experts": w.E, "top_k": w.k,
                   "inter": w.I, "routed_rows": w.T * w.k,
                   "schedule": a.schedule,
                   "minibatch_rows": ({"forward": a.minibatch_rows, "backward": a.minibatch_rows}
                                      if a.minibatch_rows else
                                      {"forward": default_minibatch(w, True),
                                       "backward": default_minibatch(w, False),
                                       "rule": "library default: two full waves of 256x256 "
                                               "tiles of the direction's first GEMM on 256 CUs "
                                               "(forward at least half the rows)"})
                   if a.schedule == "pipelined" else None},
        "roofline": main_res["roofline"],
    }
    res.update({k: v for k, v in main_res.items()
                if k not in ("value", "ms_per_step", "roofline")})
    res["schedule"] = a.schedule
    if companion:
        res["kimi_mx"] = companion
    if sweep:
        res["minibatch_sweep"] = sweep
    if decode:
        res["decode"] = decode
    if cpu:
        res["cpu_baseline"] = cpu
    del inp_main
    print(json.dumps(res), flush=True)


def _describe(w):
    return (f"{w.name}: T={w.T} tokens, top-{w.k} ({w.T * w.k} routed rows), "
            f"hidden {w.H}, {w.E} experts of intermediate {w.I}"
            + (f", shared expert {w.shared_I}" if w.shared_I else "")
            + (f", Zipf s={w.zipf_s}" if w.routing == "supplied" else ""))


def decode_bench(b, n):
    """moe_decode_fwd on the first n tokens (same weights and routing), HIP
    events on the current stream around K calls; bytes = the weights of the
    experts those tokens select (+ the shared expert), read once."""
    np, torch, m, w, a = b.np, b.torch, b.m, b.w, b.a
    inp, d = b.inp, b.d
    sh = m.Shape(n, w.H, w.E, w.k, w.I, w.shared_I, m.MOE_BF16)
    L = m.MoeLayer(sh, b.dev)
    L.prepare(d(inp["w_gate"]), d(inp["w_up"]), d(inp["w_down"]), d(inp["ws_gate"]),
              d(inp["ws_up"]), d(inp["ws_down"]))
    kw = dict(w_router=b.wr, bias=b.bias)
    if b.wr is None:
        kw = dict(topk_idx=b.idx[:n].contiguous(), topk_w=b.tw[:n].contiguous())
    xs = b.x[:n].contiguous()

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
    if b.wr is None:
        used = len(np.unique(inp["topk_idx"][:n]))
    else:
        used = len(np.unique(L.saved_tensor("topk_idx", torch.int32, (n, w.k)).cpu().numpy()))
    wbytes = (used * 3 * w.H * w.I + 3 * w.H * w.shared_I) * 2
    gbs = wbytes / (t_dec * 1e-3) / 1e9
    return {"tokens": n, "decode_ms": t_dec, "layer_fwd_ms": t_fwd, "experts_read": used,
            "weight_bytes": wbytes, "achieved_GBs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS}


if __name__ == "__main__":
    main()
