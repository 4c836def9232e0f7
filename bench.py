"""Benchmark of the NF4 LoRA linear layer (libqlora) on one MI355X.

Headline (the JSON line's `value`): forward + backward throughput in TFLOP/s
of one LLaMA-7B-shaped decoder layer's seven projections (q, k, v, o 4096 x
4096; gate, up 11008 x 4096; down 4096 x 11008) at M = 4096 tokens (batch 4 x
sequence 1024), LoRA rank 64, alpha 16, NF4 + FP8 double-quantized frozen
base, BF16 activations.  One step = for every projection: forward (saving
T = s X A^T) then backward (dX, dA, dB), 14 library calls.  Useful FLOPs per
projection = 4 M d_in d_out + 6 M r (d_in + d_out).  Before the W warm-up
steps the step runs back to back for --settle-ms (default 300 ms, reported
as settle_ms): after an idle gap the GPU's clocks need some 30-40 ms of
continuous load to settle, and the first fused-GEMM launches run 10-15 %
slower until they do.

The same line also carries, each measured in the same run:
  dropout  the headline step in training mode with LoRA dropout p = 0.05
           (the principles page's configuration), same FLOP count;
  decode   fused forward at M = 1, 4, 16 over the 7B layer in one grouped call
           per layer, scored as HBM GB/s over the packed weight bytes (NF4
           codes + FP8 scale codes + FP32 second-level scales + mean); four
           distinct quantized copies of the layer rotate so the 256 MB
           last-level cache holds none of them;
  quant    quantize and dequantize of the 7B layer's seven projections, each
           as one grouped call (quantize, dequant) and as seven single calls
           (quantize_each, dequant_each), GB/s over the algorithmic bytes (read
           FP32 W + write packed state; read packed + write BF16);
  blocked  quantize / dequantize of the 7B layer as flat arrays at first-level
           block sizes 32, 128 and 256 (groups of 256), GB/s as for quant;
  merge    LoRA merge into the restored base plus requantization of the 7B
           layer (r = 64), GB/s over packed-read + FP32 write/read + packed write;
  adamw    one clipped AdamW step (global-norm sum of squares, then the
           update with a BF16 copy) over the r = 64 adapters of one 7B layer
           (14 tensors, 5.0 M parameters) and of all 32 layers (448 tensors,
           160 M), GB/s over 34 bytes per parameter (gradient read twice,
           parameter and both moments read and written, BF16 copy written);
  stack65b forward + backward of all 560 LoRA linears of an 80-layer
           LLaMA-65B-shaped stack (hidden 8192, FFN 22016) at M = 2048, one
           layer at a time, packed weights resident in HBM;
  roofline the dominant kernel (fused dequant-GEMM), timed per launch with HIP
           events placed around it on the launch stream by the timing build
           of the library (libqlora_timed.so: the same kernels plus that
           event hook), in a pass of its own after the headline steps, which
           run on libqlora.so without events;
  peaks    the peaks this GPU reaches: a streaming read of a 4 GiB buffer and a
           loop of back-to-back BF16 MFMAs (libqlora_peaks.so), beside the
           published 8 TB/s and 2.5 PFLOP/s;
  cpu_baseline  the CPU oracle on the host cores: the headline workload on a
           token sample (extrapolated to the full step), and per configuration
           (256 x 256 layer, 7B quantize + dequantize, 7B decode at M = 1, 4,
           16, 7B training step, 65B stack) in cpu_baseline_configs.
All inputs are seeded synthetic tensors (bit_quantized_lora_quantize_amd.inputs).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

_ROOT = os.path.dirname(os.path.abspath(__file__))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

import bit_quantized_lora_quantize_amd as q  # noqa: E402
from bit_quantized_lora_quantize_amd import _lib, inputs  # noqa: E402

METRIC = "NF4-LoRA linear: eff. HBM GB/s (M<=16) & TFLOPS fwd+bwd (M=4096)"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
R, ALPHA = 64, 16.0

# HBM bytes per fused-GEMM launch (mean over the 14 launches of one training
# step), from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs scaled by a
# 1024 MB device copy (factors 2.0 and 1.0).  Valid only for the kernel
# sources with this SHA-1 (gemm_source_sha1); reported as null otherwise.
GEMM_TRAFFIC_BYTES = 273.42e6
GEMM_TRAFFIC_SHA1 = "4e508d5cfbbb20d2f09d6d2c774931ea50b1fe00"


def gemm_source_sha1():
    """SHA-1 of what decides the fused GEMM's memory traffic: gemm.hip,
    qlora_device.h and the GemmArgs declaration in qlora_kernels.h."""
    import hashlib
    import re
    csrc = os.path.join(_ROOT, "bit_quantized_lora_quantize_amd", "csrc")
    h = hashlib.sha1()
    for f in ("gemm.hip", "qlora_device.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(csrc, "qlora_kernels.h")) as fh:
        m = re.search(r"struct GemmArgs \{.*?\};", fh.read(), re.S)
    h.update(m.group(0).encode() if m else b"")
    return h.hexdigest()


def gemm_traffic():
    # counted at r = 64 on the GEMM sources of that SHA-1
    return GEMM_TRAFFIC_BYTES if gemm_source_sha1() == GEMM_TRAFFIC_SHA1 and R == 64 else None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def packed_bytes(d_out, d_in):
    return sum(q.qlora_nf4_sizes(d_out, d_in))


def useful_flops(M, d_out, d_in, r):
    return 4 * M * d_in * d_out + 6 * M * r * (d_in + d_out)


class KernelTimer:
    """Per-launch HIP events around the library's weight kernel.  The library
    records them on the stream it launches the kernel on (torch's current
    stream); elapsed times are read after the timed region synchronizes."""

    _hip = None

    def __init__(self):
        import ctypes
        if KernelTimer._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            KernelTimer._hip = hip
        self.ct = ctypes
        self.pairs = []

    def _event(self):
        ev = self.ct.c_void_p()
        assert KernelTimer._hip.hipEventCreate(self.ct.byref(ev)) == 0
        return ev

    def arm(self, tag):
        """Only inside _lib.library(_lib.TIMED_LIB_PATH)."""
        s, e = self._event(), self._event()
        q.qlora_time_next_weight_kernel(s, e)
        self.pairs.append((tag, s, e))

    def durations_ms(self, tag):
        out = []
        for t, s, e in self.pairs:
            if t != tag:
                continue
            ms = self.ct.c_float()
            assert KernelTimer._hip.hipEventElapsedTime(self.ct.byref(ms), s, e) == 0
            out.append(ms.value)
        return out

    def __del__(self):
        # through type(self): at interpreter exit the module's globals may be gone
        hip = type(self)._hip
        if hip is None:
            return
        for _, s, e in getattr(self, "pairs", []):
            hip.hipEventDestroy(s)
            hip.hipEventDestroy(e)


# ------------------------------------------------------------------ layers

class Layer:
    """Quantized weights and LoRA factors of one decoder layer."""

    def __init__(self, shapes, M, config, layer, dev, fwd_workspace=False):
        self.items = []
        for p, (name, d_out, d_in) in enumerate(shapes):
            W = inputs.weight(d_out, d_in, config, layer, device=dev, proj=p)
            w = q.qlora_quantize_nf4(W)
            del W
            A, B = inputs.lora_factors(d_out, d_in, R, config, layer, device=dev, proj=p)
            it = dict(name=name, w=w, A=A, B=B, d_out=d_out, d_in=d_in)
            if fwd_workspace:
                it["wsf"] = torch.empty(q.qlora_workspace_bytes(q.QLORA_OP_FWD, d_out, d_in, M, R),
                                        dtype=torch.uint8, device=dev)
            self.items.append(it)


class Activations:
    """Per projection shape: X, dY, outputs, saved T and workspaces, shared by
    every layer (layers run one after another on one stream)."""

    def __init__(self, shapes, M, config, dev, dropout=False):
        self.buf = {}
        fop = q.QLORA_OP_FWD_DROPOUT if dropout else q.QLORA_OP_FWD
        bop = q.QLORA_OP_BWD_DROPOUT if dropout else q.QLORA_OP_BWD
        for p, (name, d_out, d_in) in enumerate(shapes):
            key = (d_out, d_in)
            if key in self.buf:
                continue
            self.buf[key] = dict(
                X=inputs.activations(M, d_in, config, 0, inputs.T_X, device=dev, proj=p),
                dY=inputs.activations(M, d_out, config, 0, inputs.T_DY, device=dev, proj=p),
                Y=torch.empty((M, d_out), dtype=torch.bfloat16, device=dev),
                dX=torch.empty((M, d_in), dtype=torch.bfloat16, device=dev),
                dA=torch.empty((R, d_in), dtype=torch.float32, device=dev),
                dB=torch.empty((d_out, R), dtype=torch.float32, device=dev),
                T=torch.empty((M, R), dtype=torch.float32, device=dev),
                wsf=torch.empty(q.qlora_workspace_bytes(fop, d_out, d_in, M, R),
                                dtype=torch.uint8, device=dev),
                wsb=torch.empty(q.qlora_workspace_bytes(bop, d_out, d_in, M, R),
                                dtype=torch.uint8, device=dev))


def train_step(layer, acts, timer=None, p_drop=None, step=0):
    for n, it in enumerate(layer.items):
        a = acts.buf[(it["d_out"], it["d_in"])]
        if timer:
            timer.arm("fwd")
        if p_drop is None:
            q.qlora_linear_fwd(it["w"], a["X"], it["A"], it["B"], ALPHA, Y=a["Y"],
                               T_save=a["T"], workspace=a["wsf"])
        else:
            # the forward saves its keep bits for the backward (as T), so the
            # mask is generated once per step
            if "keep_rows" not in a:
                M, d_in = a["X"].shape
                m = q.Dropout(p_drop, 0).saved_mask(M, d_in, a["X"].device)
                a["keep_rows"], a["keep_cols"] = m.keep_rows, m.keep_cols
            drop = q.Dropout(p_drop, seed=0x5EED, offset=len(layer.items) * step + n,
                             keep_rows=a["keep_rows"], keep_cols=a["keep_cols"])
            q.qlora_linear_fwd_dropout(it["w"], a["X"], it["A"], it["B"], ALPHA, drop,
                                       Y=a["Y"], T_save=a["T"], workspace=a["wsf"])
        if timer:
            timer.arm("bwd")
        if p_drop is None:
            q.qlora_linear_bwd(it["w"], a["X"], a["dY"], it["A"], it["B"], ALPHA,
                               T_saved=a["T"], dX=a["dX"], dA=a["dA"], dB=a["dB"],
                               workspace=a["wsb"])
        else:
            q.qlora_linear_bwd_dropout(it["w"], a["X"], a["dY"], it["A"], it["B"], ALPHA, drop,
                                       T_saved=a["T"], dX=a["dX"], dA=a["dA"], dB=a["dB"],
                                       workspace=a["wsb"])


def timed(fn, steps, warmup):
    for _ in range(warmup):
        fn(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


# -------------------------------------------------------------- workloads

def settle(step, settle_ms):
    """Untimed steps back to back for at least settle_ms before the warm-up:
    after an idle gap the GPU's clocks take some 30-40 ms of continuous load
    to reach their steady state (the first fused-GEMM launches after idle run
    10-15 % slower), and the warm-up steps alone cover less than that."""
    n = 0
    t_end = time.perf_counter() + settle_ms * 1e-3
    while time.perf_counter() < t_end:
        step()
        torch.cuda.synchronize()
        n += 1
    return n


def bench_train7b(dev, steps, warmup, settle_ms=0.0):
    M = 4096
    log(f"7B layer fwd+bwd: M={M} r={R}; quantizing 7 projections")
    layer = Layer(inputs.LLAMA_7B, M, 3, 0, dev)
    acts = Activations(inputs.LLAMA_7B, M, 3, dev)
    torch.cuda.synchronize()
    flops = sum(useful_flops(M, d_out, d_in, R) for _, d_out, d_in in inputs.LLAMA_7B)
    n_settle = settle(lambda: train_step(layer, acts), settle_ms)
    log(f"settle: {n_settle} untimed steps in {settle_ms:.0f} ms, then {warmup} warm-up steps")
    for _ in range(warmup):
        train_step(layer, acts)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        train_step(layer, acts)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    # dominant kernel: the fused dequant-GEMM, forward and backward launches,
    # timed per launch in a pass of its own on the timing build
    timer = KernelTimer()
    with _lib.library(_lib.TIMED_LIB_PATH):
        train_step(layer, acts)
        torch.cuda.synchronize()
        for _ in range(steps):
            train_step(layer, acts, timer)
        torch.cuda.synchronize()
    gemm_flops_fwd = [2 * M * d_out * (d_in + R) for _, d_out, d_in in inputs.LLAMA_7B]
    gemm_flops_bwd = [2 * M * d_in * (d_out + R) for _, d_out, d_in in inputs.LLAMA_7B]
    dur_f = timer.durations_ms("fwd")
    dur_b = timer.durations_ms("bwd")
    fl_f = gemm_flops_fwd * steps
    fl_b = gemm_flops_bwd * steps
    ach_f = sum(fl_f) / (sum(dur_f) * 1e-3) / 1e12
    ach_b = sum(fl_b) / (sum(dur_b) * 1e-3) / 1e12
    ach = (sum(fl_f) + sum(fl_b)) / ((sum(dur_f) + sum(dur_b)) * 1e-3) / 1e12
    res = dict(elapsed=el, flops_per_step=flops, tflops=flops * steps / el / 1e12,
               ms_per_step=el / steps * 1e3,
               gemm=dict(fwd_avg_us=sum(dur_f) / len(dur_f) * 1e3,
                         bwd_avg_us=sum(dur_b) / len(dur_b) * 1e3,
                         fwd_tflops=ach_f, bwd_tflops=ach_b, tflops=ach,
                         flops_per_launch_avg=(sum(fl_f) + sum(fl_b)) / (len(fl_f) + len(fl_b)),
                         avg_launch_ms=(sum(dur_f) + sum(dur_b)) / (len(dur_f) + len(dur_b))))
    log(f"7B fwd+bwd: {res['tflops']:.1f} TFLOP/s ({res['ms_per_step']:.3f} ms/step); "
        f"fused GEMM fwd {ach_f:.1f} bwd {ach_b:.1f} TFLOP/s")
    del layer, acts
    torch.cuda.empty_cache()
    return res


def bench_dropout7b(dev, steps, warmup, p_drop=0.05):
    """The headline step with LoRA dropout p = 0.05 (training mode): mask
    generation in the forward and again in the backward, masked LoRA input,
    and the masked LoRA term of dX inside the backward GEMM."""
    M = 4096
    layer = Layer(inputs.LLAMA_7B, M, 3, 0, dev)
    acts = Activations(inputs.LLAMA_7B, M, 3, dev, dropout=True)
    torch.cuda.synchronize()
    flops = sum(useful_flops(M, d_out, d_in, R) for _, d_out, d_in in inputs.LLAMA_7B)
    for i in range(warmup):
        train_step(layer, acts, p_drop=p_drop, step=i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        train_step(layer, acts, p_drop=p_drop, step=warmup + i)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    timer = KernelTimer()
    with _lib.library(_lib.TIMED_LIB_PATH):
        train_step(layer, acts, p_drop=p_drop, step=warmup + steps)
        torch.cuda.synchronize()
        for i in range(steps):
            train_step(layer, acts, timer, p_drop=p_drop, step=warmup + steps + 1 + i)
        torch.cuda.synchronize()
    dur_b = timer.durations_ms("bwd")
    fl_b = [2 * M * d_in * (d_out + R) for _, d_out, d_in in inputs.LLAMA_7B] * steps
    res = dict(p=p_drop, tflops=flops * steps / el / 1e12, ms_per_step=el / steps * 1e3,
               bwd_gemm_avg_us=sum(dur_b) / len(dur_b) * 1e3,
               bwd_gemm_tflops=sum(fl_b) / (sum(dur_b) * 1e-3) / 1e12)
    log(f"7B fwd+bwd with LoRA dropout p={p_drop}: {res['tflops']:.1f} TFLOP/s "
        f"({res['ms_per_step']:.3f} ms/step); masked backward GEMM {res['bwd_gemm_tflops']:.1f} "
        f"TFLOP/s")
    del layer, acts
    torch.cuda.empty_cache()
    return res


def bench_decode7b(dev, steps, warmup, copies=4):
    out = {}
    scored = sum(packed_bytes(d_out, d_in) for _, d_out, d_in in inputs.LLAMA_7B)
    for M in (1, 4, 16):
        layers = [Layer(inputs.LLAMA_7B, M, 2, c, dev, fwd_workspace=True)
                  for c in range(copies)]
        xs = {}
        for c in range(copies):
            for p, (name, d_out, d_in) in enumerate(inputs.LLAMA_7B):
                xs[(c, p)] = (inputs.activations(M, d_in, 2, c, inputs.T_X, device=dev, proj=p),
                              torch.empty((M, d_out), dtype=torch.bfloat16, device=dev))
        groups = []
        for c, L in enumerate(layers):
            groups.append([q.FwdItem(it["w"], xs[(c, p)][0], it["A"], it["B"], ALPHA,
                                     xs[(c, p)][1], it["wsf"]) for p, it in enumerate(L.items)])
        torch.cuda.synchronize()
        timer = KernelTimer()
        n = max(steps, 8) * copies

        def step(i, tm=None):
            g = groups[(0 if i is None else i) % copies]
            if tm:
                tm.arm("gemv")
            q.qlora_linear_fwd_many(g, M)

        for i in range(max(warmup, 2) * copies):
            step(i)
        torch.cuda.synchronize()
        # whole calls back to back (no timing events between them), then the
        # same calls again with the weight kernel of each bracketed by events
        t0 = time.perf_counter()
        for i in range(n):
            step(i)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        with _lib.library(_lib.TIMED_LIB_PATH):
            for i in range(copies):
                step(i)
            torch.cuda.synchronize()
            for i in range(n):
                step(i, timer)
            torch.cuda.synchronize()
        durs = timer.durations_ms("gemv")
        k_avg = sum(durs) / len(durs) * 1e-3
        out[f"M{M}"] = dict(layer_us=el / n * 1e6, gbps=scored / (el / n) / 1e9,
                            gemv_us=k_avg * 1e6, gemv_gbps=scored / k_avg / 1e9,
                            gemv_frac=scored / k_avg / 1e9 / PEAK_HBM_GBS)
        log(f"decode M={M}: layer {el / n * 1e6:.1f} us = {scored / (el / n) / 1e9:.0f} GB/s; "
            f"weight kernel {k_avg * 1e6:.1f} us = {scored / k_avg / 1e9:.0f} GB/s")
        del layers, groups, xs
        torch.cuda.empty_cache()
    out["scored_bytes_per_layer"] = scored
    return out


def bench_quant7b(dev, steps, warmup):
    Ws = [inputs.weight(d_out, d_in, 1, 0, outliers=True, device=dev, proj=p)
          for p, (_, d_out, d_in) in enumerate(inputs.LLAMA_7B)]
    qs = [q.qlora_quantize_nf4(W) for W in Ws]
    outs = [torch.empty(W.shape, dtype=torch.bfloat16, device=dev) for W in Ws]
    wss = [torch.empty(q.qlora_workspace_bytes(q.QLORA_OP_QUANTIZE, *W.shape), dtype=torch.uint8,
                       device=dev) for W in Ws]
    n = sum(W.numel() for W in Ws)
    packed = sum(w.nbytes() for w in qs)
    bq = 4 * n + packed
    bd = packed + 2 * n

    # the layer's seven projections in one grouped call (the way a layer is
    # loaded), and as seven single calls
    def qstep(i, tm=None):
        if tm:
            tm.arm("q")
        q.qlora_quantize_nf4_many(Ws, outs=qs, workspaces=wss)

    def dstep(i, tm=None):
        if tm:
            tm.arm("d")
        q.qlora_dequant_bf16_many(qs, outs=outs)

    def qstep_each(i, tm=None):
        for W, w, ws in zip(Ws, qs, wss):
            if tm:
                tm.arm("q")
            q.qlora_quantize_nf4(W, out=w, workspace=ws)

    def dstep_each(i, tm=None):
        for w, o in zip(qs, outs):
            if tm:
                tm.arm("d")
            q.qlora_dequant_bf16(w, out=o)

    res = {}
    for name, fn, nbytes in (("quantize", qstep, bq), ("dequant", dstep, bd),
                             ("quantize_each", qstep_each, bq), ("dequant_each", dstep_each, bd)):
        # wall clock without timing events between the launches, then one
        # more pass with the weight kernel of every call bracketed by events
        el = timed(fn, steps, warmup) / steps
        tm = KernelTimer()
        with _lib.library(_lib.TIMED_LIB_PATH):
            fn(None)
            torch.cuda.synchronize()
            fn(None, tm)
            torch.cuda.synchronize()
        dur = tm.durations_ms(name[0])
        res[name] = dict(layer_us=el * 1e6, gbps=nbytes / el / 1e9, bytes=nbytes,
                         weight_kernel_us=sum(dur) * 1e3)
        log(f"{name} 7B layer: {el * 1e6:.1f} us = {nbytes / el / 1e9:.0f} GB/s "
            f"(weight kernel {sum(dur) * 1e3:.1f} us)")
    del Ws, qs, outs, wss
    torch.cuda.empty_cache()
    return res


def bench_blocked7b(dev, steps, warmup):
    """Quantize and dequantize the 7B layer's weights as flat arrays at other
    first-level block sizes (second-level groups of 256); algorithmic bytes
    as for the layer format, with that block size's metadata."""
    Ws = [inputs.weight(d_out, d_in, 1, 0, outliers=True, device=dev, proj=p).view(-1)
          for p, (_, d_out, d_in) in enumerate(inputs.LLAMA_7B)]
    n = sum(W.numel() for W in Ws)
    res = {}
    for block in (32, 128, 256):
        qs = [q.qlora_quantize_nf4_blocked(W, block, 256) for W in Ws]
        outs = [torch.empty(W.numel(), dtype=torch.bfloat16, device=dev) for W in Ws]
        wss = [torch.empty(q.qlora_quantize_blocked_workspace_bytes(W.numel(), block, 256),
                           dtype=torch.uint8, device=dev) for W in Ws]
        packed = sum(t.numel() * t.element_size() for b in qs
                     for t in (b.codes, b.scale_codes, b.scale2, b.scale_mean))

        def qstep(i, Ws=Ws, qs=qs, wss=wss, block=block):
            for W, b, ws in zip(Ws, qs, wss):
                q.qlora_quantize_nf4_blocked(W, block, 256, out=b, workspace=ws)

        def dstep(i, qs=qs, outs=outs):
            for b, o in zip(qs, outs):
                q.qlora_dequant_bf16_blocked(b, out=o)

        eq = timed(qstep, steps, warmup) / steps
        ed = timed(dstep, steps, warmup) / steps
        res[f"B{block}"] = dict(quantize_us=eq * 1e6, quantize_gbps=(4 * n + packed) / eq / 1e9,
                                dequant_us=ed * 1e6, dequant_gbps=(packed + 2 * n) / ed / 1e9,
                                bits_per_weight=packed * 8 / n)
        log(f"blocked B1={block}: quantize {eq * 1e6:.1f} us = {(4 * n + packed) / eq / 1e9:.0f} "
            f"GB/s; dequant {ed * 1e6:.1f} us = {(packed + 2 * n) / ed / 1e9:.0f} GB/s; "
            f"{packed * 8 / n:.4f} bits/weight")
        del qs, outs, wss
    del Ws
    torch.cuda.empty_cache()
    return res


def bench_merge7b(dev, steps, warmup):
    """LoRA merge (FP32 Wh + s B A, FP64 evaluation) and requantization of the
    7B layer's seven projections, r = 64.  Bytes: packed state read (0.516
    B/weight) + FP32 merged weight written and read back by the quantizer (8
    B/weight) + the new packed state written (0.516 B/weight)."""
    items = []
    for p, (_, d_out, d_in) in enumerate(inputs.LLAMA_7B):
        W = inputs.weight(d_out, d_in, 5, 0, device=dev, proj=p)
        w = q.qlora_quantize_nf4(W)
        del W
        A, B = inputs.lora_factors(d_out, d_in, R, 5, 0, device=dev, proj=p)
        Wm = torch.empty((d_out, d_in), dtype=torch.float32, device=dev)
        wo = q.NF4Weight.empty(d_out, d_in, dev)
        ws = torch.empty(q.qlora_workspace_bytes(q.QLORA_OP_QUANTIZE, d_out, d_in),
                         dtype=torch.uint8, device=dev)
        items.append((w, A, B, Wm, wo, ws))
    n = sum(d_out * d_in for _, d_out, d_in in inputs.LLAMA_7B)
    packed = sum(it[0].nbytes() for it in items)
    nbytes = 2 * packed + 8 * n

    def step(i):
        for w, A, B, Wm, wo, ws in items:
            q.qlora_merge_nf4(w, A, B, ALPHA, W_merged=Wm, out=wo, workspace=ws)

    el = timed(step, steps, warmup) / steps
    res = dict(layer_us=el * 1e6, gbps=nbytes / el / 1e9, bytes=nbytes,
               fp64_gflops=2 * R * n / el / 1e9)
    log(f"merge + requantize 7B layer: {el * 1e6:.1f} us = {nbytes / el / 1e9:.0f} GB/s")
    del items
    torch.cuda.empty_cache()
    return res


def bench_adamw7b(dev, steps, warmup):
    """Clipped AdamW steps over the 7B adapters (r = 64): one layer's 14
    tensors, then the 448 tensors of 32 layers.  Per step: zero the FP64
    accumulator, sum of squares, update.  34 bytes per parameter."""
    res = {}
    for name, layers in (("layer", 1), ("model32", 32)):
        params = []
        for layer in range(layers):
            for p, (_, d_out, d_in) in enumerate(inputs.LLAMA_7B):
                for n in (R * d_in, d_out * R):
                    g, m, v = inputs.optimizer_state(n, 6, layer=(7 * layer + p) % 16,
                                                     device=dev)
                    params.append(q.AdamwParam(
                        torch.empty(n, device=dev).normal_(0, 0.02), g, m, v,
                        torch.empty(n, dtype=torch.bfloat16, device=dev)))
        ps = q.AdamwParamSet(params)
        ps.sumsq_workspace()
        acc = torch.zeros(1, dtype=torch.float64, device=dev)
        n_total = sum(t.param.numel() for t in params)

        def step(i):
            acc.zero_()
            q.qlora_grad_sumsq(ps, acc)
            q.qlora_adamw_step(ps, lr=2e-4, weight_decay=0.01, step=(i or 0) + 1,
                               grad_sumsq=acc, max_grad_norm=0.3)

        el = timed(step, steps, warmup) / steps
        nbytes = 34 * n_total
        res[name] = dict(params=n_total, tensors=len(params), us=el * 1e6,
                         gbps=nbytes / el / 1e9)
        log(f"adamw {name}: {len(params)} tensors, {n_total / 1e6:.1f} M params: "
            f"{el * 1e6:.1f} us = {nbytes / el / 1e9:.0f} GB/s")
        del params, ps
        torch.cuda.empty_cache()
    return res


def bench_stack65b(dev, steps, warmup):
    M = 2048
    log(f"65B stack: {inputs.LLAMA_65B_LAYERS} layers x 7, M={M}; quantizing")
    t0 = time.perf_counter()
    layers = [Layer(inputs.LLAMA_65B, M, 4, l, dev) for l in range(inputs.LLAMA_65B_LAYERS)]
    acts = Activations(inputs.LLAMA_65B, M, 4, dev)
    torch.cuda.synchronize()
    resident = sum(it["w"].nbytes() for L in layers for it in L.items)
    log(f"65B stack ready in {time.perf_counter() - t0:.1f} s; packed weights "
        f"{resident / 1e9:.2f} GB resident")
    flops = inputs.LLAMA_65B_LAYERS * sum(useful_flops(M, d_out, d_in, R)
                                          for _, d_out, d_in in inputs.LLAMA_65B)

    def step(i):
        for L in layers:
            train_step(L, acts)

    el = timed(step, steps, warmup)
    res = dict(tflops=flops * steps / el / 1e12, s_per_step=el / steps,
               resident_packed_gb=resident / 1e9, flops_per_step=flops)
    log(f"65B stack fwd+bwd: {res['tflops']:.1f} TFLOP/s ({res['s_per_step']:.3f} s/step)")
    del layers, acts
    torch.cuda.empty_cache()
    return res


class Peaks:
    """The measurement kernels of libqlora_peaks.so."""

    def __init__(self):
        import ctypes
        path = os.path.join(os.path.dirname(_lib.LIB_PATH), "libqlora_peaks.so")
        if not os.path.exists(path):
            raise ImportError(f"libqlora_peaks.so is not built ({path})")
        L = ctypes.CDLL(path)
        P, I = ctypes.c_void_p, ctypes.c_int
        L.qlora_peak_stream_read.argtypes = [P, ctypes.c_int64, P, I, P]
        L.qlora_peak_mfma.argtypes = [P, I, I, P]
        self.L = L

    @staticmethod
    def _events_ms(fn, reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps

    def measure(self, dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        nbytes = 4 << 30
        buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=dev)
        sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
        best_read = 0.0
        for wgs in (1024, 2048, 4096, 8192):
            def run(wgs=wgs):
                assert self.L.qlora_peak_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), wgs,
                                                     stream) == 0
            ms = self._events_ms(run, 5)
            best_read = max(best_read, nbytes / (ms * 1e-3) / 1e9)
        del buf
        fsink = torch.zeros(4096 * 256, dtype=torch.float32, device=dev)
        iters, best_mfma = 1024, 0.0
        for wgs in (512, 1024, 2048):
            def run(wgs=wgs):
                assert self.L.qlora_peak_mfma(fsink.data_ptr(), wgs, iters, stream) == 0
            ms = self._events_ms(run, 3)
            flops = wgs * 4 * iters * 4 * 2 * 32 * 32 * 16
            best_mfma = max(best_mfma, flops / (ms * 1e-3) / 1e12)
        torch.cuda.empty_cache()
        log(f"measured peaks: streaming read {best_read:.0f} GB/s, BF16 MFMA loop "
            f"{best_mfma:.1f} TFLOP/s")
        return dict(hbm_read_gbs=round(best_read, 1), mfma_bf16_tflops=round(best_mfma, 1),
                    read_kernel="16-byte loads over a 4 GiB buffer, best of 1024..8192 workgroups",
                    mfma_kernel="v_mfma_f32_32x32x16_bf16, 4 independent accumulators per "
                                "wavefront, best of 512..2048 workgroups")


def _median_time(fn, runs):
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return sorted(ts)[len(ts) // 2]


def cpu_baselines(tokens=128, stack_tokens=32):
    """The oracle (plain C, FP64 products, OpenMP over rows) on the host
    cores, per configuration; quantization of the inputs untimed except in
    the quantize + dequantize configuration.  Returns (the headline
    workload's entry, all entries)."""
    import numpy as np
    import oracle
    cores = oracle.num_threads()
    out = {}
    f32 = lambda t: t.float().numpy()

    def prep(d_out, d_in, config, layer=0, proj=0, outliers=False):
        W = inputs.weight(d_out, d_in, config, layer, outliers=outliers, proj=proj).numpy()
        st = oracle.quantize_nf4(W)
        Wh = oracle.bf16_bits_to_f32(oracle.dequant_bf16(*st, W.size)).reshape(d_out, d_in)
        return W, Wh

    # 256 x 256, M = 16, r = 8: quantize, dequantize, forward and backward
    log("cpu baseline: 256 x 256 layer")
    W, _ = prep(256, 256, 0)
    A, B = (f32(t) for t in inputs.lora_factors(256, 256, 8, 0))
    X = f32(inputs.activations(16, 256, 0, 0, inputs.T_X))
    dY = f32(inputs.activations(16, 256, 0, 0, inputs.T_DY))

    def small():
        st = oracle.quantize_nf4(W)
        Wh = oracle.bf16_bits_to_f32(oracle.dequant_bf16(*st, W.size)).reshape(256, 256)
        oracle.linear_fwd(Wh, X, A, B, 2.0)
        oracle.linear_bwd(Wh, X, dY, A, B, 2.0)

    t_all = _median_time(small, 3)
    oracle.set_num_threads(1)
    t_one = _median_time(small, 3)
    oracle.set_num_threads(cores)
    out["layer256_M16_r8"] = dict(ms=round(t_all * 1e3, 3), ms_1core=round(t_one * 1e3, 3),
                                  cores=cores, runs="median of 3",
                                  work="quantize + dequantize + fwd + bwd")

    # 7B layer: quantize + dequantize (weights with outliers)
    log("cpu baseline: 7B layer quantize + dequantize")
    Ws = [inputs.weight(d_out, d_in, 1, 0, outliers=True, proj=p).numpy()
          for p, (_, d_out, d_in) in enumerate(inputs.LLAMA_7B)]
    n = sum(w.size for w in Ws)
    packed = sum(packed_bytes(d_out, d_in) for _, d_out, d_in in inputs.LLAMA_7B)
    states = [oracle.quantize_nf4(w) for w in Ws]
    tq = _median_time(lambda: [oracle.quantize_nf4(w) for w in Ws], 3)
    td = _median_time(lambda: [oracle.dequant_bf16(*st, w.size) for st, w in zip(states, Ws)], 3)
    out["llama7b_quant_dequant"] = dict(
        quantize_ms=round(tq * 1e3, 1), quantize_gbs=round((4 * n + packed) / tq / 1e9, 3),
        dequant_ms=round(td * 1e3, 1), dequant_gbs=round((packed + 2 * n) / td / 1e9, 3),
        cores=cores, runs="median of 3")
    del Ws, states

    # 7B layer decode forward, M = 1, 4, 16 (all seven projections)
    log("cpu baseline: 7B layer decode forward, M = 1, 4, 16")
    r = R
    layer7 = []
    for p, (_, d_out, d_in) in enumerate(inputs.LLAMA_7B):
        _, Wh = prep(d_out, d_in, 2, 0, p)
        A, B = (f32(t) for t in inputs.lora_factors(d_out, d_in, r, 2, 0, proj=p))
        layer7.append((Wh, A, B, d_in))
    dec = {}
    for M in (1, 4, 16):
        xs = [f32(inputs.activations(M, d_in, 2, 0, inputs.T_X, proj=p))
              for p, (_, _, _, d_in) in enumerate(layer7)]
        t = _median_time(lambda: [oracle.linear_fwd(Wh, X, A, B, ALPHA / r)
                                  for (Wh, A, B, _), X in zip(layer7, xs)], 3)
        dec[f"M{M}"] = dict(layer_ms=round(t * 1e3, 2), gbs=round(packed / t / 1e9, 4))
    out["llama7b_decode"] = dict(dec, cores=cores, runs="median of 3",
                                 gbs_over="packed weight bytes, as the GPU figure")
    del layer7

    # 7B layer training step on a token sample (the headline workload)
    log(f"cpu baseline: 7B layer fwd + bwd on {tokens} tokens")
    total_t, flops = 0.0, 0
    for p, (_, d_out, d_in) in enumerate(inputs.LLAMA_7B):
        _, Wh = prep(d_out, d_in, 3, 0, p)
        A, B = (f32(t) for t in inputs.lora_factors(d_out, d_in, r, 3, 0, proj=p))
        X = f32(inputs.activations(tokens, d_in, 3, 0, inputs.T_X, proj=p))
        dY = f32(inputs.activations(tokens, d_out, 3, 0, inputs.T_DY, proj=p))
        t0 = time.perf_counter()
        oracle.linear_fwd(Wh, X, A, B, ALPHA / r)
        oracle.linear_bwd(Wh, X, dY, A, B, ALPHA / r)
        total_t += time.perf_counter() - t0
        flops += useful_flops(tokens, d_out, d_in, r)
    head = dict(value=flops / total_t / 1e12, unit="TFLOP/s", cores=cores, kind="oracle",
                sample=f"fwd+bwd (Y, dX, dA, dB) of the 7 LLaMA-7B projections on {tokens} of "
                       f"the 4096 tokens, r={r}, FP64 accumulation, quantization untimed; "
                       f"{total_t:.1f} s of CPU time; the full 4096-token step extrapolates "
                       f"to {total_t * 4096 / tokens:.0f} s")
    out["llama7b_train_M4096"] = dict(tflops=round(head["value"], 5),
                                      sample_tokens=tokens, sample_s=round(total_t, 2),
                                      step_s_extrapolated=round(total_t * 4096 / tokens, 1),
                                      cores=cores, label="extrapolated (token sample x 4096 / "
                                                         "sample)")

    # 65B stack: layer 0 on a token sample, extrapolated to 2048 tokens x 80 layers
    log(f"cpu baseline: 65B layer 0 fwd + bwd on {stack_tokens} tokens")
    total_t, flops = 0.0, 0
    for p, (_, d_out, d_in) in enumerate(inputs.LLAMA_65B):
        _, Wh = prep(d_out, d_in, 4, 0, p)
        A, B = (f32(t) for t in inputs.lora_factors(d_out, d_in, r, 4, 0, proj=p))
        X = f32(inputs.activations(stack_tokens, d_in, 4, 0, inputs.T_X, proj=p))
        dY = f32(inputs.activations(stack_tokens, d_out, 4, 0, inputs.T_DY, proj=p))
        t0 = time.perf_counter()
        oracle.linear_fwd(Wh, X, A, B, ALPHA / r)
        oracle.linear_bwd(Wh, X, dY, A, B, ALPHA / r)
        total_t += time.perf_counter() - t0
        flops += useful_flops(stack_tokens, d_out, d_in, r)
        del Wh
    step_s = total_t * (2048 / stack_tokens) * inputs.LLAMA_65B_LAYERS
    out["llama65b_stack_M2048"] = dict(tflops=round(flops / total_t / 1e12, 5),
                                       sample="layer 0, 7 projections", sample_tokens=stack_tokens,
                                       sample_s=round(total_t, 2),
                                       step_s_extrapolated=round(step_s, 0), cores=cores,
                                       label="extrapolated (layer 0 token sample x 2048 / "
                                             "sample x 80 layers)")
    return head, out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed steps back to back for this long before the warm-up steps "
                         "(clock ramp after idle)")
    ap.add_argument("--skip", default="", help="comma list of: dropout,decode,quant,blocked,merge,adamw,stack65b,peaks,cpu")
    ap.add_argument("--cpu-tokens", type=int, default=1024)
    ap.add_argument("--cpu-stack-tokens", type=int, default=128)
    ap.add_argument("--rank", type=int, default=64,
                    help="LoRA rank r of every leg (the headline figure is quoted at 64)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="first run one device-to-device copy of this many MB (a plain copy "
                         "kernel of known size, for scaling hardware byte counters)")
    args = ap.parse_args()
    global R
    R = args.rank
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    skip = set(s for s in args.skip.split(",") if s)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q.lib()
    log(f"device {torch.cuda.get_device_name(dev)}; steps={args.steps} warmup={args.warmup}")
    if args.copy_mb > 0:
        n = args.copy_mb * 1000 * 1000 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.copy_mb} MB read + {args.copy_mb} MB written")
        del src, dst

    train = bench_train7b(dev, args.steps, args.warmup, args.settle_ms)
    extra = {}
    if "dropout" not in skip:
        extra["dropout_7b"] = bench_dropout7b(dev, args.steps, args.warmup)
    if "decode" not in skip:
        extra["decode_7b"] = bench_decode7b(dev, args.steps, args.warmup)
    if "quant" not in skip:
        extra["quant_7b"] = bench_quant7b(dev, max(3, args.steps // 2), 1)
    if "blocked" not in skip:
        extra["blocked_7b"] = bench_blocked7b(dev, max(3, args.steps // 2), 1)
    if "merge" not in skip:
        extra["merge_7b"] = bench_merge7b(dev, max(3, args.steps // 2), 1)
    if "adamw" not in skip:
        extra["adamw_7b"] = bench_adamw7b(dev, args.steps, args.warmup)
    if "stack65b" not in skip:
        extra["stack_65b"] = bench_stack65b(dev, max(1, min(args.steps, 2)), 1)
    peaks = None if "peaks" in skip else Peaks().measure(dev)
    cpu, cpu_cfg = (None, None) if "cpu" in skip else cpu_baselines(args.cpu_tokens, args.cpu_stack_tokens)

    g = train["gemm"]
    line = {
        "metric": METRIC,
        "value": round(train["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(train["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"llama7b_layer_7proj_fwd_bwd_M4096_r{R}",
                   "tokens": 4096, "rank": R, "lora_alpha": ALPHA,
                   "projections": [f"{n} {o}x{i}" for n, o, i in inputs.LLAMA_7B],
                   "quant": "NF4 block 64 + FP8 E4M3FN double quant block 256",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(g["tflops"], 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(g["tflops"] / PEAK_BF16_TFLOPS, 4), "traffic": gemm_traffic(),
                     "kernel": "k_gemm (fused dequant-GEMM, fwd and bwd)",
                     "avg_launch_us": round(g["avg_launch_ms"] * 1e3, 2),
                     "fwd_avg_us": round(g["fwd_avg_us"], 2), "bwd_avg_us": round(g["bwd_avg_us"], 2),
                     "fwd_tflops": round(g["fwd_tflops"], 2), "bwd_tflops": round(g["bwd_tflops"], 2)},
        "cpu_baseline": cpu,
        "cpu_baseline_configs": cpu_cfg,
        "peaks": peaks,
    }
    if peaks:
        line["roofline"]["measured_peak"] = peaks["mfma_bf16_tflops"]
        line["roofline"]["frac_of_measured_peak"] = round(g["tflops"] / peaks["mfma_bf16_tflops"], 4)
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
