#!/usr/bin/env python3
"""Benchmark of the sparse MoE experts forward pass on one MI355X.

One step = one pass of the whole hot path over one batch: router logits (x . Wr^T) + softmax
top-k (moe_route), expert grouping (moe_permute), fp8 activation quantisation (fp8 layers), gate/up
grouped GEMM + SwiGLU and down grouped GEMM with the fused unpermute/weighting epilogue
(moe_experts_forward), and the k-slot combine (moe_combine). Synthetic seeded inputs, already
resident in HBM.

The JSON line's value is the Mixtral-shaped prefill layer (T=4096 tokens, d=4096, f=14336, E=8,
top-2, bf16 with fp32 accumulation) in active TFLOP/s, with the roofline of its dominant kernel
(the gate/up GEMM, MFMA-bound) timed with HIP events on the launch stream. The same line carries
the Mixtral-shaped decode layer (T=32, weight streaming, HBM-bound), the skewed 128-expert bf16
layer (T=16384, d=2048, f=768, k=8), the DeepSeek-V3-shaped fine-grained FP8 layer (T=8192,
d=7168, f=2048, E=256, k=8) with fp32 and with UE8M0 block scales, each with its own roofline
object, and the CPU oracle timed on a bounded token sample as a reference baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
METRIC = "MoE layer active TFLOP/s (prefill) + tokens/s (decode), % MFMA/HBM peak"
CSRC = os.path.join(ROOT, "mixture_experts_ffn_softmax_amd", "csrc")
GEMM_SOURCES = ("common.h", "gemm_bf16.hip")
DECODE_SOURCES = ("common.h", "decode_bf16.hip")
FP8_SOURCES = ("common.h", "gemm_fp8.hip")
# counter summaries (profiles/) of the gate/up GEMM of the other workloads, by workload name
OTHER_TRAFFIC = {
    "skewed_bf16_T16384_d2048_f768_E128_k8": ("gemm_bf16_gate_up_skewed_128e_hbm_bytes.txt",
                                              GEMM_SOURCES),
    "dsv3_fp8_T8192_d7168_f2048_E256_k8": ("gemm_fp8_gate_up_dsv3_f32_scales_hbm_bytes.txt",
                                           FP8_SOURCES),
    "dsv3_fp8_T8192_d7168_f2048_E256_k8_ue8m0": ("gemm_fp8_gate_up_dsv3_ue8m0_hbm_bytes.txt",
                                                 FP8_SOURCES),
}


def source_code_text(text):
    """C++ source text with // and /* */ comments removed and whitespace runs collapsed, so that
    editing a comment does not change what identifies a kernel build."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(files):
    """sha256 over the code of the named kernel sources, comments and layout left out (identifies
    the kernel build a counter run measured)."""
    import hashlib
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(CSRC, name), encoding="utf-8") as fh:
            h.update(name.encode() + b"\0" + source_code_text(fh.read()).encode())
    return h.hexdigest()


def measured_traffic(summary_name, files):
    """HBM bytes per dispatch (FETCH + WRITE, copy-calibrated) from a counter summary under
    profiles/, or None when the summary is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", summary_name)
    try:
        with open(path) as fh:
            fields = dict(line.split(":", 1) for line in fh if ":" in line and not line.startswith(" "))
    except OSError:
        return None
    fields = {k.strip(): v.strip() for k, v in fields.items()}
    if fields.get("source_sha256") != source_digest(files):
        return None
    try:
        return int(float(fields["hbm_bytes_per_dispatch"]))
    except (KeyError, ValueError):
        return None


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


class Layer:
    """Device buffers for one MoE layer workload and a step() that enqueues the whole path:
    moe_route (given logits, or the fp32 router GEMM), moe_permute, fp8_quantize_act (fp8
    layers), moe_experts_forward, moe_combine."""

    def __init__(self, moe, spec, x, W, n_ev_steps, logits=None, Wr=None, scales=None,
                 scale_fmt="f32"):
        import torch
        self.moe, self.spec = moe, spec
        self.lib = moe.load_library()
        dev = "cuda"
        T, d, f, E, k = spec.T, spec.d, spec.f, spec.E, spec.k
        P = T * k
        Wg, Wu, Wd = W
        self.keep = [x, Wg, Wu, Wd, logits, Wr, scales]
        act = moe.MOE_F32 if spec.dtype == "f32" else moe.MOE_BF16
        wdt = {"f32": moe.MOE_F32, "bf16": moe.MOE_BF16, "fp8": moe.MOE_FP8_E4M3,
               "fp4": moe.MOE_FP4_E2M1}[spec.dtype]
        lowp = spec.dtype in ("fp8", "fp4")   # e4m3 activations with block scales
        ydt = moe.MOE_F32 if spec.dtype == "f32" else moe.MOE_BF16
        tdt = torch.float32 if ydt == moe.MOE_F32 else torch.bfloat16
        self.logits = logits if logits is not None else torch.empty((T, E), dtype=torch.float32,
                                                                   device=dev)
        self.ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.counts = torch.empty(E, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.sp = torch.empty(P, dtype=torch.int32, device=dev)
        self.pp = torch.empty(P, dtype=torch.int32, device=dev)
        pw = self.lib.moe_permute_workspace_size(T, k, E)
        self.pws = torch.empty(max(pw, 1), dtype=torch.uint8, device=dev)
        xact = moe.MOE_FP8_E4M3 if lowp else act
        ew = self.lib.moe_experts_workspace_size(T, d, f, E, k, xact, wdt)
        self.ews = torch.empty(ew, dtype=torch.uint8, device=dev)
        self.y = torch.empty((T, k, d), dtype=tdt, device=dev)
        self.out = torch.empty((T, d), dtype=tdt, device=dev)
        # per-projection timing: HIP events on the stream the library launches on (torch's
        # current stream, which self.stream is), around a gate/up-only and a down-only call
        self.events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
                       for _ in range(n_ev_steps)]
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
        self._quant = None
        x_in, xs = x, None
        ue = scale_fmt == "ue8m0"
        self._quant_fn = self.lib.fp8_quantize_act_ue8m0 if ue else self.lib.fp8_quantize_act
        if lowp:
            self.xq = torch.empty((T, d), dtype=torch.uint8, device=dev)
            self.xs = torch.empty((T, d // 128), dtype=torch.uint8 if ue else torch.float32,
                                  device=dev)
            self._quant = (p(x), moe.MOE_BF16, T, d, 128, None, p(self.xq), p(self.xs),
                           self.stream)
            x_in, xs = self.xq, self.xs
        sg = su = sd = None
        if scales is not None:
            sg, su, sd = scales
        self.args = moe.moe_experts_args(
            T, d, f, E, k, xact, wdt, ydt, moe.MOE_Y_SLOTS, x_in.data_ptr(),
            xs.data_ptr() if xs is not None else None, Wg.data_ptr(), Wu.data_ptr(),
            Wd.data_ptr(), sg.data_ptr() if sg is not None else None,
            su.data_ptr() if su is not None else None, sd.data_ptr() if sd is not None else None,
            self.offsets.data_ptr(), self.sp.data_ptr(), self.w.data_ptr(), self.y.data_ptr(),
            self.ews.data_ptr(), self.ews.numel(),
            moe.MOE_SCALE_UE8M0 if ue else moe.MOE_SCALE_F32, moe.MOE_PHASE_ALL)
        if logits is None:
            self._route = (None, p(x), act, p(Wr), T, d, E, k, p(self.logits), p(self.ids),
                           p(self.w), self.stream)
        else:
            self._route = (p(logits), None, act, None, T, d, E, k, None, p(self.ids), p(self.w),
                           self.stream)
        self._perm = (p(self.ids), T, k, E, p(self.counts), p(self.offsets), p(self.sp),
                      p(self.pp), None, 0, None, 0, None, None, p(self.pws), self.pws.numel(),
                      self.stream)
        self._comb = (p(self.y), ydt, moe.MOE_Y_SLOTS, None, None, T, k, d, p(self.out), ydt,
                      self.stream)

    def step(self, ev_index=None):
        lib, chk = self.lib, self.moe._check
        chk(lib.moe_route(*self._route))
        chk(lib.moe_permute(*self._perm))
        if self._quant is not None:
            chk(self._quant_fn(*self._quant))
        if ev_index is None:
            self.args.phase = self.moe.MOE_PHASE_ALL
            chk(lib.moe_experts_forward(ctypes.byref(self.args), self.stream))
        else:
            # the same work as one MOE_PHASE_ALL call, split so that events bracket each projection
            ev = self.events[ev_index]
            ev[0].record()
            self.args.phase = self.moe.MOE_PHASE_GATE_UP
            chk(lib.moe_experts_forward(ctypes.byref(self.args), self.stream))
            ev[1].record()
            self.args.phase = self.moe.MOE_PHASE_DOWN
            chk(lib.moe_experts_forward(ctypes.byref(self.args), self.stream))
            ev[2].record()
        chk(lib.moe_combine(*self._comb))

    def phase_ms(self, phase, reps):
        """Mean duration (ms) of one projection phase run ``reps`` times back to back between two
        HIP events on the launch stream (the decode kernels stream their weights from HBM on
        every call: the weights are far larger than the on-chip caches)."""
        import torch
        lib, chk = self.lib, self.moe._check
        self.args.phase = phase
        chk(lib.moe_experts_forward(ctypes.byref(self.args), self.stream))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            chk(lib.moe_experts_forward(ctypes.byref(self.args), self.stream))
        e1.record()
        torch.cuda.synchronize()
        self.args.phase = self.moe.MOE_PHASE_ALL
        return e0.elapsed_time(e1) / reps

    def kernel_ms(self, n):
        """Mean duration (ms) of the gate/up phase (its tile-table launch included) and of the
        down phase over the first n event-timed steps."""
        g1 = [e[0].elapsed_time(e[1]) for e in self.events[:n]]
        g2 = [e[1].elapsed_time(e[2]) for e in self.events[:n]]
        return sum(g1) / n, sum(g2) / n


def time_steps(layer, steps, warmup, events=True):
    """Wall time of ``steps`` steps after ``warmup``. events=True records the per-kernel HIP events
    inside the timed steps; each record sits between two kernels on the stream and costs a few
    microseconds, so short steps are timed without them (see kernel_pass)."""
    import torch
    for _ in range(warmup):
        layer.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        layer.step(ev_index=i if events else None)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def kernel_pass(layer, steps):
    """Per-kernel durations (gate/up incl. any h quantisation, down) over ``steps`` further steps
    with HIP events."""
    import torch
    for i in range(steps):
        layer.step(ev_index=i)
    torch.cuda.synchronize()
    return layer.kernel_ms(steps)


def vendor_gemm(spec, iters=20):
    """The vendor library on dense bf16 products with the FLOPs of the layer's two grouped GEMMs
    (P = T*k rows, gate and up as one 2f-wide weight): context for the grouped kernels, not part
    of the path."""
    import torch
    P, d, f = spec.P, spec.d, spec.f
    out = {}
    for name, (M, N, K) in (("gate_up", (P, 2 * f, d)), ("down", (P, d, f))):
        a = torch.randn((M, K), device="cuda").to(torch.bfloat16)
        w = (torch.randn((N, K), device="cuda") * 0.02).to(torch.bfloat16)
        for _ in range(3):
            y = torch.nn.functional.linear(a, w)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            y = torch.nn.functional.linear(a, w)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        out[name] = {"M": M, "N": N, "K": K, "ms": round(ms, 4), "tflops": round(tf, 1),
                     "pct_bf16_peak": round(100 * tf / BF16_PEAK_TFLOPS, 2)}
        log("vendor dense %s %dx%dx%d: %.3f ms, %.1f TFLOP/s" % (name, M, N, K, ms, tf))
        del a, w, y
    torch.cuda.empty_cache()
    return out


def host_cpu():
    """Model name, logical CPUs available to this process, and the OpenMP thread setting."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count() or 1
    return model, nproc, os.environ.get("OMP_NUM_THREADS")


def cpu_baseline(spec, x_np, Wr_np, W_np, seconds):
    """The oracle, as it stands, on the first n tokens of the workload (routing included)."""
    import numpy as np
    import oracle
    ex = oracle.Experts(*W_np)
    model, nproc, omp = host_cpu()
    threads = int(omp) if omp else nproc   # the oracle's OpenMP loops use this many threads

    def run(n):
        xs = np.ascontiguousarray(x_np[:n])
        t0 = time.perf_counter()
        lg = oracle.router_logits(xs, Wr_np)
        ids, w = oracle.route(lg, spec.k)
        oracle.moe_forward(xs, ex, ids, w)
        return time.perf_counter() - t0

    n = 8
    dt = run(n)
    n2 = int(min(spec.T, max(n, n * seconds / max(dt, 1e-3))))
    if n2 > n:
        n, dt = n2, run(n2)
    toks = n / dt
    return {
        "value": round(spec.active_flops() / spec.T * toks / 1e12, 6),
        "unit": "TFLOP/s",
        "tokens_per_s": round(toks, 2),
        "seconds": round(dt, 2),
        "cores": threads,
        "cpu_model": model,
        "nproc": nproc,
        "omp_num_threads": omp,
        "kind": "oracle",
        "sample": "first %d of the %d tokens of %s (%d token-expert pairs): router logits, "
                  "top-k routing, experts and combine, fp64 per-token loop" % (
                      n, spec.T, spec.name, n * spec.k),
    }


def expert_histogram(counts):
    """Per-expert load summary: rows of the busiest and least busy expert, empty experts, and the
    share of all pairs taken by the busiest expert and by the 8 busiest."""
    import numpy as np
    c = np.sort(np.asarray(counts, np.int64))[::-1]
    tot = max(int(c.sum()), 1)
    return {"max_rows": int(c[0]), "min_rows": int(c[-1]), "empty": int((c == 0).sum()),
            "nonempty": int((c > 0).sum()), "max_share": round(float(c[0]) / tot, 4),
            "top8_share": round(float(c[:8].sum()) / tot, 4)}


def lowp_weights(moe, synth, spec, fmts, fp4=False):
    """Expert weights of an fp8 workload on the device, quantised there from the generator's fp32
    masters (16 experts at a time): {fmt: ((W_gate, W_up, W_down), (s_gate, s_up, s_down))} for
    each fmt in fmts ("f32" / "ue8m0" block scales), or {"fp4": ...} E2M1 with MX scales."""
    import numpy as np
    import torch

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    out = {f: ([], []) for f in (("fp4",) if fp4 else fmts)}
    for which in ("gate", "up", "down"):
        rows, cols = (spec.f, spec.d) if which != "down" else (spec.d, spec.f)
        bufs = {}
        for f in out:
            if f == "fp4":
                bufs[f] = (torch.empty((spec.E, rows, cols // 2), dtype=torch.uint8, device="cuda"),
                           torch.empty((spec.E, rows, cols // 32), dtype=torch.uint8, device="cuda"))
            else:
                bufs[f] = (torch.empty((spec.E, rows, cols), dtype=torch.uint8, device="cuda"),
                           torch.empty((spec.E, rows // 128, cols // 128), device="cuda",
                                       dtype=torch.uint8 if f == "ue8m0" else torch.float32))
        for e0 in range(0, spec.E, 16):
            m = up(synth.gen_expert_weight(spec.with_(dtype="fp8"), which,
                                           experts=range(e0, min(e0 + 16, spec.E))))
            for f, (q, sc) in bufs.items():
                if f == "fp4":
                    qq, ss = moe.fp4_quantize_weight_mx(m, tiled=True)
                else:
                    qq, ss = moe.fp8_quantize_weight(m, scale_fmt=f)
                q[e0:e0 + 16] = qq
                sc[e0:e0 + 16] = ss
            del m
        for f, (q, sc) in bufs.items():
            out[f][0].append(q)
            out[f][1].append(sc)
    return {f: (tuple(w), tuple(sc)) for f, (w, sc) in out.items()}


FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 MFMA


def measure_other(moe, synth, spec, steps, warmup, weights=None, scale_fmt="f32", name=None):
    """Times one workload with given router logits and returns its figures, with the roofline of
    its gate/up GEMM (the kernel that takes the most time). ``weights``: device (W, S) of a
    low-precision layer (lowp_weights), with scale_fmt "f32", "ue8m0" or "fp4" (E2M1, MX)."""
    import numpy as np
    import torch

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    t0 = time.perf_counter()
    x = up(synth.gen_x(spec))
    logits = up(synth.gen_logits(spec))
    scales = None
    if weights is not None:
        W, scales = weights
        if scale_fmt == "fp4":
            spec = spec.with_(dtype="fp4")
            scale_fmt = "ue8m0"
    else:
        W = [up(synth.gen_expert_weight(spec, n)) for n in ("gate", "up", "down")]
    name = name or spec.name
    log("%s inputs ready in %.1fs" % (name, time.perf_counter() - t0))
    layer = Layer(moe, spec, x, tuple(W), steps, logits=logits, scales=scales,
                  scale_fmt=scale_fmt)
    el = time_steps(layer, steps, warmup, events=False)
    g1, g2 = kernel_pass(layer, steps)
    counts = layer.counts.cpu().numpy()
    touched = int((counts > 0).sum())
    wbytes = {"f32": 4, "bf16": 2, "fp8": 1, "fp4": 0.5 + 1 / 32}[spec.dtype]
    w_bytes = touched * 3 * spec.d * spec.f * wbytes
    ms = el / steps * 1e3
    tflops = spec.active_flops() / (ms * 1e-3) / 1e12
    g1_flops = 4.0 * spec.P * spec.d * spec.f
    r = {
        "workload": name, "ms_per_step": round(ms, 4),
        "active_tflops": round(tflops, 2),
        "tokens_per_s": round(spec.T / (ms * 1e-3), 1),
        "gate_up_ms": round(g1, 4), "down_ms": round(g2, 4),
        "gate_up_tflops": round(g1_flops / (g1 * 1e-3) / 1e12, 2),
        "down_tflops": round(2.0 * spec.P * spec.d * spec.f / (g2 * 1e-3) / 1e12, 2),
        "weight_GBps_layer": round(w_bytes / (ms * 1e-3) / 1e9, 1),
        "experts_touched": touched,
        "expert_histogram": expert_histogram(counts),
    }
    if spec.dtype in ("fp8", "fp4"):
        # gate/up roofline: the weights of the touched experts (+ their scales), the x codes and
        # scales, and the h codes and scales it writes, against 8 TB/s; its FLOPs against the fp8
        # peak. The larger of the two ideal times is the bound.
        P, d, f = spec.P, spec.d, spec.f
        sc_w = 2 * f * d / 32 if spec.dtype == "fp4" else 2 * (f // 128) * (d // 128) * 4
        g1_bytes = touched * (2 * f * d * wbytes + sc_w) + spec.T * d * (1 + 4 / 128) + \
            P * f * (1 + 4 / 128)
        t_hbm = g1_bytes / (HBM_PEAK_GBS * 1e9)
        t_mfma = g1_flops / (FP8_PEAK_TFLOPS * 1e12)
        hbm = {"bound": "hbm", "achieved": round(g1_bytes / (g1 * 1e-3) / 1e9, 1),
               "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(g1_bytes / (g1 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        mfma = {"bound": "mfma", "achieved": round(g1_flops / (g1 * 1e-3) / 1e12, 2),
                "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(g1_flops / (g1 * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4)}
        roof = dict(hbm if t_hbm >= t_mfma else mfma)
        roof["kernel"] = "gemm_fp8_kernel<gate_up> (gate/up grouped GEMM + SwiGLU + h quantisation)"
        roof["other_roof_frac"] = (mfma if t_hbm >= t_mfma else hbm)["frac"]
        roof["traffic"] = measured_traffic(*OTHER_TRAFFIC[name]) if name in OTHER_TRAFFIC else None
        r["roofline"] = roof
        r["pct_fp8_peak"] = round(100 * tflops / FP8_PEAK_TFLOPS, 2)
        ideal = max(w_bytes / (HBM_PEAK_GBS * 1e9), spec.active_flops() / (FP8_PEAK_TFLOPS * 1e12))
        r["pct_hbm_peak"] = round(100 * w_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)
        r["layer_roofline_frac"] = round(ideal / (ms * 1e-3), 4)
    elif spec.dtype == "bf16":
        r["roofline"] = {"kernel": "gemm_bf16_kernel<gate_up> (gate/up grouped GEMM + SwiGLU)",
                         "bound": "mfma", "achieved": r["gate_up_tflops"],
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(r["gate_up_tflops"] / BF16_PEAK_TFLOPS, 4),
                         "traffic": (measured_traffic(*OTHER_TRAFFIC[name])
                                     if name in OTHER_TRAFFIC else None)}
        r["pct_bf16_peak"] = round(100 * tflops / BF16_PEAK_TFLOPS, 2)
        r["layer_roofline_frac"] = round(
            spec.active_flops() / (BF16_PEAK_TFLOPS * 1e12) / (ms * 1e-3), 4)
    log("%s: %.3f ms/step, %.1f TFLOP/s (gate/up %.3f ms, down %.3f ms)" % (
        name, ms, r["active_tflops"], g1, g2))
    del layer
    torch.cuda.empty_cache()
    return r


def measure_decode_fp8(moe, synth, W, Wr, steps, warmup, scale_fmt, fp4=False):
    """The Mixtral-shaped decode layer with its bf16 weights quantised to e4m3 (128x128 blocks,
    fp32 or UE8M0 scales), or with fp4=True to E2M1 with MX scales (one e8m0 byte per row per 32
    channels), on the device: the weight-streaming kernels."""
    import torch
    dspec = synth.MIXTRAL_DECODE.with_(dtype="fp4" if fp4 else "fp8")
    name = "mixtral_decode_%s_T%d_d%d_f%d_E%d_k%d%s" % (
        "fp4" if fp4 else "fp8", dspec.T, dspec.d, dspec.f, dspec.E, dspec.k,
        "_mx" if fp4 else ("_ue8m0" if scale_fmt == "ue8m0" else ""))
    Q, S = [], []
    for w in W:
        if fp4:
            q, s_ = moe.fp4_quantize_weight_mx(w, tiled=True)
        else:
            q, s_ = moe.fp8_quantize_weight(w, scale_fmt=scale_fmt)
        Q.append(q)
        S.append(s_)
    xd = torch.from_numpy(synth.gen_x(synth.MIXTRAL_DECODE).view("int16")).cuda().view(torch.bfloat16)
    layer = Layer(moe, dspec, xd, tuple(Q), steps, Wr=Wr, scales=tuple(S), scale_fmt=scale_fmt)
    el = time_steps(layer, steps, warmup, events=False)
    g1 = layer.phase_ms(moe.MOE_PHASE_GATE_UP, steps)
    g2 = layer.phase_ms(moe.MOE_PHASE_DOWN, steps)
    touched = int((layer.counts.cpu().numpy() > 0).sum())
    ms = el / steps * 1e3
    per_w = 0.5 + 1 / 32 if fp4 else 1.0   # streamed bytes per weight (E2M1 codes + MX scales)
    wb = touched * 3 * dspec.d * dspec.f * per_w
    r = {"workload": name, "ms_per_step": round(ms, 4),
         "tokens_per_s": round(dspec.T / (ms * 1e-3), 1),
         "gate_up_ms": round(g1, 4), "down_ms": round(g2, 4),
         "gate_up_weight_GBps": round(touched * 2 * dspec.d * dspec.f * per_w / (g1 * 1e-3) / 1e9,
                                      1),
         "weight_GBps_layer": round(wb / (ms * 1e-3) / 1e9, 1), "experts_touched": touched}
    log("%s: %.3f ms/step, %.0f tokens/s; gate/up %.3f ms (%.0f GB/s of weights), down "
        "%.3f ms (incl. h quantisation)" % (name, ms, r["tokens_per_s"], g1,
                                            r["gate_up_weight_GBps"], g2))
    del layer, Q, S
    torch.cuda.empty_cache()
    return r


def measure_fused(moe, synth, W, Wr, steps, warmup, fmt):
    """The Mixtral-shaped decode layer through moe_fused_forward (one routing kernel with the router
    GEMM, top-k and x quantisation; no permutation), weights bf16, e4m3 with UE8M0 scales
    ("ue8m0") or E2M1 with MX scales ("fp4"), quantised on the device."""
    import torch
    spec = synth.MIXTRAL_DECODE
    T, d, f, E, k = spec.T, spec.d, spec.f, spec.E, spec.k
    if fmt == "bf16":
        Q, S, wdt = list(W), [None] * 3, moe.MOE_BF16
    elif fmt == "fp4":
        Q, S = zip(*[moe.fp4_quantize_weight_mx(w, tiled=True) for w in W])
        wdt = moe.MOE_FP4_E2M1
    else:
        Q, S = zip(*[moe.fp8_quantize_weight(w, scale_fmt="ue8m0") for w in W])
        wdt = moe.MOE_FP8_E4M3
    x = torch.from_numpy(synth.gen_x(spec).view("int16")).cuda().view(torch.bfloat16)
    out = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lib = moe.load_library()
    ws = torch.empty(lib.moe_fused_workspace_size(T, d, f, E, k, wdt, moe.MOE_BF16),
                     dtype=torch.uint8, device="cuda")
    p = lambda t: t.data_ptr() if t is not None else None
    args = moe.moe_fused_args(T, d, f, E, k, moe.MOE_BF16, wdt,
                              moe.MOE_SCALE_UE8M0 if fmt != "bf16" else moe.MOE_SCALE_F32,
                              p(x), None, p(Wr), None, *(p(q) for q in Q), *(p(s_) for s_ in S),
                              p(out), moe.MOE_BF16, p(ids), p(w), p(ws), ws.numel())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ref = ctypes.byref(args)

    def run(n):
        for _ in range(n):
            moe._check(lib.moe_fused_forward(ref, stream))
    run(warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    name = "mixtral_decode_fused_%s_T%d_d%d_f%d_E%d_k%d" % (fmt, T, d, f, E, k)
    log("%s: %.3f ms/step, %.0f tokens/s" % (name, ms, T / (ms * 1e-3)))
    del Q, S, ws
    torch.cuda.empty_cache()
    return {"workload": name, "ms_per_step": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1)}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=25.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the skewed 128-expert and DeepSeek-V3-shaped fp8 workloads")
    ap.add_argument("--others", default="skewed,dsv3_fp8,dsv3_fp8_ue8m0",
                    help="which of the skewed / DeepSeek-V3-shaped workloads to time (comma list "
                         "of skewed, dsv3_fp8, dsv3_fp8_ue8m0)")
    ap.add_argument("--report", default="",
                    help="also time the fp8 / FP4 and fused decode variants, the DeepSeek-V3-shaped "
                         "layer with FP4 experts and the tiny fp32 layer; write every workload's "
                         "figures to this JSON file")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="first time the vendor library (torch.nn.functional.linear, hipBLASLt) on "
                         "dense bf16 products of the Mixtral-shaped GEMMs' sizes, for context")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run a plain fp32 copy kernel (out = in * 1) over this many MiB, "
                         "3 times, to calibrate HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_ffn_softmax_amd as moe
    import synth

    torch.cuda.set_device(0)
    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log("copy probe: %d MiB read + %d MiB written per launch" % (args.copy_probe_mib,
                                                                    args.copy_probe_mib))
        del src, dst
    vendor = vendor_gemm(synth.MIXTRAL_PREFILL) if args.vendor_gemm else None
    spec = synth.MIXTRAL_PREFILL
    T, d, f, E, k = spec.T, spec.d, spec.f, spec.E, spec.k
    log("generating %s inputs" % spec.name)
    t0 = time.perf_counter()

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    x_np = synth.gen_x(spec)
    Wr_np = synth.gen_router_weight(spec)
    W_np = [synth.gen_expert_weight(spec, n) for n in ("gate", "up", "down")]
    x, Wr = up(x_np), up(Wr_np)
    Wg, Wu, Wd = (up(a) for a in W_np)
    log("inputs ready in %.1fs" % (time.perf_counter() - t0))

    if args.no_prefill:
        args.steps = 1
    layer = Layer(moe, spec, x, (Wg, Wu, Wd), max(args.steps, 1), Wr=Wr)
    el = time_steps(layer, args.steps, args.warmup)
    ms = el / args.steps * 1e3
    g1_ms, g2_ms = layer.kernel_ms(args.steps)
    flops = spec.active_flops()
    tflops = flops / (el / args.steps) / 1e12
    g1_flops = 4.0 * spec.P * d * f
    g1_tflops = g1_flops / (g1_ms * 1e-3) / 1e12
    counts = layer.counts.cpu().numpy()
    log("prefill: %.3f ms/step, %.1f TFLOP/s; gate/up %.3f ms (%.1f TFLOP/s), down %.3f ms"
        % (ms, tflops, g1_ms, g1_tflops, g2_ms))

    result = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": spec.name, "T": T, "d": d, "f": f, "E": E, "k": k,
            "tokens_per_s": round(T / (el / args.steps), 1),
            "pct_bf16_peak": round(100 * tflops / BF16_PEAK_TFLOPS, 2),
            "expert_rows_min_max": [int(counts.min()), int(counts.max())],
            "gate_up_ms": round(g1_ms, 4), "down_ms": round(g2_ms, 4),
            "down_tflops": round(2.0 * spec.P * d * f / (g2_ms * 1e-3) / 1e12, 2),
        },
        "roofline": {
            "kernel": "gemm_bf16_kernel<gate_up> (gate/up grouped GEMM + SwiGLU)",
            "bound": "mfma", "achieved": round(g1_tflops, 2), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(g1_tflops / BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic("gemm_bf16_gate_up_mixtral_prefill_hbm_bytes.txt",
                                        GEMM_SOURCES),
        },
    }
    if vendor is not None:
        result["vendor_dense_gemm"] = vendor
    del layer
    torch.cuda.empty_cache()

    if not args.no_decode:
        dspec = synth.MIXTRAL_DECODE
        xd = up(synth.gen_x(dspec))
        dl = Layer(moe, dspec, xd, (Wg, Wu, Wd), args.decode_steps, Wr=Wr)
        eld = time_steps(dl, args.decode_steps, 5, events=False)
        dms = eld / args.decode_steps * 1e3
        # per projection: each phase repeated back to back (events between the two phases of one
        # step can land before the first phase's last workgroups finish)
        d1 = dl.phase_ms(moe.MOE_PHASE_GATE_UP, args.decode_steps)
        d2 = dl.phase_ms(moe.MOE_PHASE_DOWN, args.decode_steps)
        dcounts = dl.counts.cpu().numpy()
        touched = int((dcounts > 0).sum())
        w_bytes_gu = touched * 2 * f * d * 2
        w_bytes_dn = touched * d * f * 2
        gbs1 = w_bytes_gu / (d1 * 1e-3) / 1e9
        gbs2 = w_bytes_dn / (d2 * 1e-3) / 1e9
        layer_gbs = (w_bytes_gu + w_bytes_dn) / (dms * 1e-3) / 1e9
        log("decode: %.3f ms/step, %.0f tokens/s; gate/up %.3f ms (%.0f GB/s), down %.3f ms "
            "(%.0f GB/s)" % (dms, dspec.T / (eld / args.decode_steps), d1, gbs1, d2, gbs2))
        result["decode"] = {
            "workload": dspec.name,
            "tokens_per_s": round(dspec.T / (eld / args.decode_steps), 1),
            "ms_per_step": round(dms, 4),
            "layer_weight_GBps": round(layer_gbs, 1),
            "pct_hbm_peak": round(100 * layer_gbs / HBM_PEAK_GBS, 2),
            "experts_touched": touched,
            "gate_up_ms": round(d1, 4), "down_ms": round(d2, 4),
            "roofline": {
                "kernel": "decode_stream_kernel (weight-streaming gate/up GEMM + SwiGLU)",
                "bound": "hbm", "achieved": round(gbs1, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs1 / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic("decode_bf16_gate_up_mixtral_decode_hbm_bytes.txt",
                                            DECODE_SOURCES),
            },
            "roofline_down": {
                "kernel": "decode_stream_down_kernel (weight-streaming down GEMM + weighted slots)",
                "bound": "hbm", "achieved": round(gbs2, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs2 / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic("decode_bf16_down_mixtral_decode_hbm_bytes.txt",
                                            DECODE_SOURCES),
            },
        }
        del dl

    rep = []
    if args.report:
        rep.append(result.get("decode"))
        for fmt in ("f32", "ue8m0"):
            rep.append(measure_decode_fp8(moe, synth, (Wg, Wu, Wd), Wr, max(args.decode_steps, 5),
                                          5, fmt))
        rep.append(measure_decode_fp8(moe, synth, (Wg, Wu, Wd), Wr, max(args.decode_steps, 5), 5,
                                      "ue8m0", fp4=True))
        for fmt in ("bf16", "ue8m0", "fp4"):
            rep.append(measure_fused(moe, synth, (Wg, Wu, Wd), Wr, max(args.decode_steps, 5), 5,
                                     fmt))
    del Wg, Wu, Wd
    torch.cuda.empty_cache()

    # The skewed 128-expert layer and the DeepSeek-V3-shaped fine-grained FP8 layer (its own
    # fp32 128x128 block scales, and the same masters with UE8M0 scales) are part of every run.
    others = [] if args.no_others else [w for w in args.others.split(",") if w]
    osteps = max(args.steps, 5)
    if "skewed" in others:
        result["skewed"] = measure_other(moe, synth, synth.SKEWED_128E, osteps, args.warmup)
    fmts = tuple(f for f, w in (("f32", "dsv3_fp8"), ("ue8m0", "dsv3_fp8_ue8m0")) if w in others)
    if fmts:
        t0 = time.perf_counter()
        wq = lowp_weights(moe, synth, synth.DSV3_FP8, fmts)
        log("%s weights quantised on the device in %.1fs" % (synth.DSV3_FP8.name,
                                                                time.perf_counter() - t0))
        if "f32" in wq:
            result["dsv3_fp8"] = measure_other(moe, synth, synth.DSV3_FP8, osteps, args.warmup,
                                               weights=wq.pop("f32"), scale_fmt="f32")
        if "ue8m0" in wq:
            result["dsv3_fp8_ue8m0"] = measure_other(
                moe, synth, synth.DSV3_FP8, osteps, args.warmup, weights=wq.pop("ue8m0"),
                scale_fmt="ue8m0", name=synth.DSV3_FP8.name + "_ue8m0")
        del wq
        torch.cuda.empty_cache()
    if args.report:
        rep += [result[w] for w in ("skewed", "dsv3_fp8", "dsv3_fp8_ue8m0") if w in result]
        w4 = lowp_weights(moe, synth, synth.DSV3_FP8, (), fp4=True)
        rep.append(measure_other(moe, synth, synth.DSV3_FP8, max(args.steps, 5), args.warmup,
                                 weights=w4.pop("fp4"), scale_fmt="fp4",
                                 name="dsv3_fp4_T8192_d7168_f2048_E256_k8_mx"))
        del w4
        torch.cuda.empty_cache()
        rep.append(measure_other(moe, synth, synth.TINY_F32, max(args.steps, 5), args.warmup))
        with open(args.report, "w") as fh:
            json.dump({"prefill": {k: result[k] for k in ("value", "ms_per_step", "config",
                                                          "roofline")},
                       "others": rep}, fh, indent=1)

    if not args.no_cpu_baseline:
        log("timing the CPU oracle (~%.0fs)" % args.cpu_seconds)
        result["cpu_baseline"] = cpu_baseline(spec, x_np, Wr_np, W_np, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
