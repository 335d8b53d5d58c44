#!/usr/bin/env python3
"""Benchmark of the transposed-convolution / pooling hot path on one MI355X.

A step is one pass of the whole path over its full-size synthetic workloads,
inputs already resident in HBM:
  fused3d_f32   ConvTranspose3d(3->16,k3,s2,p1) -> x0.5 -> AvgPool3d(2) -> +bias -> x1.0
                on [128,3,16,32,32] fp32 -> [128,16,15,31,31]
  avgpool3d     AvgPool3d(k3,s2,p1), divisor 27, [16,32,128,128,256] -> [16,32,64,64,128]
  convT1d       ConvTranspose1d(32->64,k5,s1,p0,d3) [32,32,131072] -> [32,64,131084]
  fused3d_bf16  the fused chain 32->64 with bf16 x and w, [16,32,16,32,32] -> [16,64,15,31,31]

Prints ONE JSON line: value = algorithmic HBM bytes of a step / step time
(GB/s), per-op ms / GB/s / GFLOP/s, the roofline of the kernel that takes the
most time (timed live with HIP events on the launch stream), and the CPU oracle
timed on a bounded sample of the same workloads.

Every op is cold by construction: it cycles through enough copies of its
input and output buffers (at least 4, more than 512 MB in all, and more than
512 MB of inputs alone) that no call
finds them in the 256 MB Infinity Cache; `ms_warm` repeats one buffer set.
Beside the 8 TB/s peak, each op's GB/s is also given as a fraction of a plain
1 GiB device copy measured in the same run (`copy_GB_s`), and `write_GB_s`
gives the rate of a write-only stream of non-constant data, the ceiling of the
write-dominated fused ops.  The small fused workload [2,3,8,16,16] is timed
per call (launch-bound) outside the step.

  python bench.py [--steps K] [--warmup W] [--ops a,b] [--no-cpu-baseline]
  python bench.py --ops copy        # plain 1 GiB device copy (counter calibration)
  python bench.py --ops fused3d_f32,unfused3d_f32   # fusion vs materialising the
                                    # [128,16,31,63,63] pre-pool tensor, then a 2-pool
  python bench.py --summarize-trace DIR [--ops a,b]  # rocprofv3 --kernel-trace CSVs -> table
                                    # (--ops: the profiled run's ops, for kernels shared by ops)
  python bench.py --summarize-counters FETCH WRITE   # rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
                                    # CSVs -> table + profiles/traffic.json
  python bench.py --summarize-pmc DIR [DIR ...]      # any rocprofv3 --pmc CSVs -> table +
                                    # profiles/counters.json (MFMA busy, VALU/SALU per MFMA)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_F32_PEAK_TFLOPS = 157.3   # dense fp32 matrix
MFMA_BF16_PEAK_TFLOPS = 2500.0 # dense bf16 matrix

OP_SOURCES = {
    "fused3d_f32": "fused3d_f32.hip",
    "avgpool3d": "avgpool3d.hip",
    "convT1d": "convT1d_f32.hip",
    "fused3d_bf16": "fused3d_bf16.hip",
    "unfused3d_f32": "generic.hip",
    "convT1d_bf16": "convT1d_bf16.hip",
    "avgpool3d_bf16": "avgpool3d.hip",
    "fused3d_general": "fused3d_f32.hip",
    "avgpool3d_nopad": "avgpool3d.hip",
    "convT1d_general": "convT1d_f32.hip",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# Kernels as rocprofv3 names them -> (op or kernel key, source file,
# algorithmic bytes of one launch at the bench workload).  The bytes are the
# same figures make_ops() computes from the tensors.
ORACLE_MIN_S = 2.5          # seconds of oracle time per op in the CPU baseline

KERNELS = [
    # the slab kernel's output_padding=1 instantiation (W = 32, 7 rows per task)
    # serves the fused3d_general workload; its other instantiations fused3d_f32
    ("fused3d_f32_slab_kernel<6, 4, 32, 7, 1>", "fused3d_general", "fused3d_f32.hip", 159388864),
    ("fused3d_f32_slab_kernel", "fused3d_f32", "fused3d_f32.hip", 143258752),
    # bf16 pool kernels first: the fp32 ones share the name prefix
    ("avgpool3d_k3s2p1_vec_kernel<unsigned short", "avgpool3d_bf16", "avgpool3d.hip", 4831838208),
    ("avgpool3d_k3s2p1_elem_kernel<unsigned short", "avgpool3d_bf16", "avgpool3d.hip", 4831838208),
    # count_include_pad=False instantiations (the include-pad template argument
    # false; the vector kernel's column-group count follows it)
    ("avgpool3d_k3s2p1_vec_kernel<float, false, false", "avgpool3d_nopad", "avgpool3d.hip", 9663676416),
    ("avgpool3d_k3s2p1_vec_kernel<float, true, false", "avgpool3d_nopad", "avgpool3d.hip", 9663676416),
    ("avgpool3d_k3s2p1_elem_kernel<float, false>", "avgpool3d_nopad", "avgpool3d.hip", 9663676416),
    ("avgpool3d_k3s2p1_", "avgpool3d", "avgpool3d.hip", 9663676416),
    # the stride-2 polyphase kernel first: it shares the fp32 prefix
    ("convT1d_f32_poly_kernel", "convT1d_general", "convT1d_f32.hip", 2684477696),
    ("convT1d_f32", "convT1d", "convT1d_f32.hip", 1610752000),
    ("fused3d_bf16_kernel", "fused3d_bf16", "fused3d_bf16.hip", 75931904),
    ("convT1d_bf16_kernel", "convT1d_bf16", "convT1d_bf16.hip", 1342296064),
    ("convT3d_s2_kernel", "convT3d_s2", "convT3d_s2.hip", 1033106496),
    ("avgpool3d_generic_kernel", "avgpool3d_generic", "generic.hip", 1126023168),
    ("fused3d_generic_kernel", "fused3d_general", "generic.hip", 159388864),
    ("fused3d_weff_kernel", "fused3d_general", "generic.hip", 159388864),
    ("convT1d_generic_kernel", "convT1d_general", "generic.hip", 2684477696),
    ("convT1d_residue_kernel", "convT1d_general", "generic.hip", 2684477696),
]


def kernel_key(name, ops=None):
    """(key, source, algorithmic bytes) of a kernel as rocprofv3 names it.  A
    kernel that serves several ops (the fp32 slab kernel) resolves to the op
    among `ops`, the ops of the profiled run, when they are given."""
    hits = [(sub, key, src, nbytes) for sub, key, src, nbytes in KERNELS
            if sub in name and (ops is None or key not in OP_SOURCES or key in ops)]
    if not hits:
        return None
    if ops is not None and len({h[1] for h in hits if h[0] == hits[0][0] and h[1] in ops}) > 1:
        AMBIGUOUS.add(name)                  # two profiled ops launch this kernel
        return None
    return hits[0][1:]


# kernels that two ops of one profiled run share: their dispatches cannot be told
# apart by name, so the summaries leave them out (profile such ops in runs of their own)
AMBIGUOUS = set()


def _report_ambiguous():
    for name in sorted(AMBIGUOUS):
        print(f"\nleft out: `{name}` is launched by more than one of the profiled ops; "
              "profile those ops in separate runs")


def source_hash(op, src=None):
    p = os.path.join(ROOT, "transposed_conv_pooling_amd", "csrc", src or OP_SOURCES[op])
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def measured_traffic(op):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when absent or taken on a different version of the kernel source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p)).get(op)
    except (OSError, ValueError):
        return None
    if not t or t.get("source_sha256_16") != source_hash(op):
        return None
    return t.get("bytes_per_launch")


# ---------------------------------------------------------------- workloads --
COLD_BYTES = 512 << 20     # twice the 256 MB Infinity Cache


def rotation_count(set_bytes, input_bytes=None):
    """Buffer sets an op cycles through so that no call finds its inputs or
    outputs left in the 256 MB Infinity Cache by an earlier call: one set when
    a single set's traffic is larger than 512 MB; else at least 4 sets, more
    than 512 MB in all, and more than 512 MB of the inputs alone (some kernels'
    non-temporal stores leave no output in the cache, but every input read is
    cached, so a rotation whose inputs fit the cache would find each input
    still there when its turn came again)."""
    if set_bytes > COLD_BYTES:
        return 1
    n = max(4, COLD_BYTES // set_bytes + 1)
    if input_bytes:
        n = max(n, COLD_BYTES // input_bytes + 1)
    return n


class Op:
    """One operation of the step.  call(bufs) launches it on one buffer set;
    run() launches it on the next set in rotation (cold by construction),
    run_warm() always on the first set (inputs and outputs cache-resident
    when they fit)."""

    def __init__(self, name, call, sets, alg_bytes, flops, bound, peak, inputs, oracle_sample):
        self.name, self.call, self.sets = name, call, sets
        self.alg_bytes, self.flops = alg_bytes, flops
        self.bound, self.peak = bound, peak
        self.inputs = inputs
        self.oracle_sample = oracle_sample    # () -> (seconds, fraction of the op)
        self._i = 0
        # arithmetic type of the products: the bf16 contractions multiply bf16
        # operands on the matrix cores (fp32 accumulation); every other op,
        # bf16 pooling included, computes in fp32
        self.arith = "bf16" if name in ("fused3d_bf16", "convT1d_bf16") else "f32"

    def run(self):
        bufs = self.sets[self._i % len(self.sets)]
        self._i += 1
        self.call(*bufs)

    def run_warm(self):
        self.call(*self.sets[0])


def bf16_label(wl):
    """Workload label for the bf16-data variant of an fp32 workload."""
    return wl.description.rsplit(" ", 1)[0] + " bf16"


def make_ops(names, dev):
    import torch

    import synth
    import transposed_conv_pooling_amd as ct

    ops = []

    def nbytes(*ts):
        return int(sum(t.numel() * t.element_size() for t in ts))

    def rotate(*ts):
        """Buffer sets [(t0, t1, ...)]: the given tensors first, then copies
        (inputs) or fresh allocations (outputs share shapes) up to the
        rotation count of their total size and of the input t0."""
        n = rotation_count(nbytes(*ts), nbytes(ts[0]))
        return [tuple(ts)] + [tuple(t.clone() for t in ts) for _ in range(n - 1)]

    if "fused3d_f32" in names:
        wl = synth.WORKLOADS["c2"]
        log(f"inputs: {wl.description}")
        t = synth.make_inputs(wl)
        x, w, b = (torch.from_numpy(t[k]).to(dev) for k in ("x", "w", "bias"))
        out = torch.empty((128, 16, 15, 31, 31), dtype=torch.float32, device=dev)

        def call(x, out, w=w, b=b):
            ct.ct_convT3d_scale_pool_bias(x, w, None, b, 0.5, 1.0, out=out)

        def sample(t=t):
            import oracle
            t0 = time.perf_counter()
            oracle.convT3d_scale_pool_bias(t["x"], t["w"], None, t["bias"], 0.5, 1.0)
            return time.perf_counter() - t0, 1.0, "all 128 batch items"

        ops.append(Op("fused3d_f32", call, rotate(x, out), nbytes(x, w, b, out),
                      2 * out.numel() * 3 * 8, "hbm", HBM_PEAK_GBS,
                      [wl.description], sample))

    if "avgpool3d" in names:
        wl = synth.WORKLOADS["c3"]
        log(f"inputs: {wl.description} (8.6 GB host generation)")
        xh = synth.normal(wl.seed, synth.STREAM_X, wl.x_shape)
        x = torch.from_numpy(xh).to(dev)
        out = torch.empty((16, 32, 64, 64, 128), dtype=torch.float32, device=dev)

        def call(x, out):
            ct.ct_avgpool3d(x, 3, 2, 1, True, out=out)

        def sample(xh=xh):
            import oracle
            k = 128
            t0 = time.perf_counter()
            oracle.avgpool3d(xh.reshape(512, 128, 128, 256)[:k], 3, 2, 1, True)
            return time.perf_counter() - t0, k / 512.0, f"{k} of 512 (n,c) slices"

        ops.append(Op("avgpool3d", call, rotate(x, out), nbytes(x, out), 27 * out.numel(), "hbm",
                      HBM_PEAK_GBS, [wl.description], sample))

    if "convT1d" in names:
        wl = synth.WORKLOADS["c4"]
        log(f"inputs: {wl.description}")
        t = synth.make_inputs(wl)
        x, w = torch.from_numpy(t["x"]).to(dev), torch.from_numpy(t["w"]).to(dev)
        out = torch.empty((32, 64, 131084), dtype=torch.float32, device=dev)

        def call(x, out, w=w):
            ct.ct_convT1d(x, w, None, 1, 0, 3, out=out)

        def sample(t=t):
            import oracle
            n = 8
            t0 = time.perf_counter()
            oracle.convT1d(t["x"][:n], t["w"], None, 1, 0, 3)
            return time.perf_counter() - t0, n / 32.0, f"{n} of 32 batch items"

        flops = 2 * 32 * 32 * 131072 * 5 * 64
        ops.append(Op("convT1d", call, rotate(x, out), nbytes(x, w, out), flops, "mfma",
                      MFMA_F32_PEAK_TFLOPS, [wl.description], sample))

    if "fused3d_bf16" in names:
        wl = synth.WORKLOADS["c5"]
        log(f"inputs: {wl.description}")
        t = synth.make_inputs(wl)
        x = torch.from_numpy(t["x_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
        w = torch.from_numpy(t["w_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
        b = torch.from_numpy(t["bias"]).to(dev)
        out = torch.empty((16, 64, 15, 31, 31), dtype=torch.float32, device=dev)

        def call(x, out, w=w, b=b):
            ct.ct_convT3d_scale_pool_bias(x, w, None, b, 0.5, 1.0, out=out)

        def sample(t=t):
            import oracle
            t0 = time.perf_counter()
            oracle.convT3d_scale_pool_bias(t["x"], t["w"], None, t["bias"], 0.5, 1.0)
            return time.perf_counter() - t0, 1.0, "all 16 batch items"

        ops.append(Op("fused3d_bf16", call, rotate(x, out), nbytes(x, w, b, out), 2 * out.numel() * 32 * 8,
                      "hbm", HBM_PEAK_GBS, [wl.description], sample))

    if "convT1d_bf16" in names:
        # the same dilated ConvTranspose1d with bf16 x and w (fp32 output)
        wl = synth.WORKLOADS["c4"]
        log(f"inputs: {wl.description} in bf16")
        t = synth.make_inputs(wl)
        xb, wb = synth.to_bf16_bits(t["x"]), synth.to_bf16_bits(t["w"])
        x = torch.from_numpy(xb.reshape(t["x"].shape).view(np.int16)).to(dev).view(torch.bfloat16)
        w = torch.from_numpy(wb.reshape(t["w"].shape).view(np.int16)).to(dev).view(torch.bfloat16)
        out = torch.empty((32, 64, 131084), dtype=torch.float32, device=dev)

        def call(x, out, w=w):
            ct.ct_convT1d(x, w, None, 1, 0, 3, out=out)

        def sample(xb=xb, wb=wb, shape=t["x"].shape, wshape=t["w"].shape):
            import oracle
            n = 8
            xf = synth.bf16_bits_to_f32(xb).reshape(shape)
            wf = synth.bf16_bits_to_f32(wb).reshape(wshape)
            t0 = time.perf_counter()
            oracle.convT1d(xf[:n], wf, None, 1, 0, 3)
            return time.perf_counter() - t0, n / 32.0, f"{n} of 32 batch items"

        flops = 2 * 32 * 32 * 131072 * 5 * 64
        ops.append(Op("convT1d_bf16", call, rotate(x, out), nbytes(x, w, out), flops, "hbm", HBM_PEAK_GBS,
                      [bf16_label(wl)], sample))

    if "avgpool3d_bf16" in names:
        # the large pooling shape with bf16 data (bf16 means of fp32 sums)
        wl = synth.WORKLOADS["c3"]
        log(f"inputs: {wl.description} in bf16 (8.6 GB host generation)")
        xb = synth.to_bf16_bits(synth.normal(wl.seed, synth.STREAM_X, wl.x_shape))
        x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
        out = torch.empty((16, 32, 64, 64, 128), dtype=torch.bfloat16, device=dev)

        def call(x, out):
            ct.ct_avgpool3d(x, 3, 2, 1, True, out=out)

        def sample(xb=xb):
            import oracle
            k = 128
            xf = synth.bf16_bits_to_f32(xb.reshape(512, 128, 128, 256)[:k])
            t0 = time.perf_counter()
            oracle.avgpool3d(xf, 3, 2, 1, True)
            return time.perf_counter() - t0, k / 512.0, f"{k} of 512 (n,c) slices"

        ops.append(Op("avgpool3d_bf16", call, rotate(x, out), nbytes(x, out), 27 * out.numel(), "hbm",
                      HBM_PEAK_GBS, [bf16_label(wl)], sample))

    if "unfused3d_f32" in names:
        # The chain without fusion: ConvTranspose3d writes the full pre-pool
        # tensor, a separate 2-pool reads it back.  (The scale / bias steps
        # would add further passes over the pooled tensor; they are left out,
        # so this is a lower bound on the unfused chain's time.)
        wl = synth.WORKLOADS["c2"]
        log(f"inputs: {wl.description} (unfused)")
        t = synth.make_inputs(wl)
        x, w = (torch.from_numpy(t[k]).to(dev) for k in ("x", "w"))
        y = torch.empty((128, 16, 31, 63, 63), dtype=torch.float32, device=dev)
        out = torch.empty((128, 16, 15, 31, 31), dtype=torch.float32, device=dev)

        def call(x, y, out, w=w):
            ct.ct_convT3d(x, w, None, 2, 1, 0, out=y)
            ct.ct_avgpool3d(y, 2, 2, 0, True, out=out)

        def sample(t=t):
            import oracle
            n = 8
            t0 = time.perf_counter()
            oracle.avgpool3d(oracle.convT3d(t["x"][:n], t["w"], None, 2, 1, 0), 2, 2, 0, True)
            return time.perf_counter() - t0, n / 128.0, f"{n} of 128 batch items"

        ops.append(Op("unfused3d_f32", call, rotate(x, y, out), nbytes(x, w, y, y, out), 2 * y.numel() * 3 * 27 // 8,
                      "hbm", HBM_PEAK_GBS, [wl.description + ", unfused"], sample))

    if "fused3d_general" in names:
        # the general gather kernel on the full-size fused workload with a
        # conv bias and output_padding=1 (pre-pool 32x64x64, pooled 16x32x32)
        wl = synth.WORKLOADS["c2"]
        log(f"inputs: {wl.description}, conv bias, output_padding=1")
        t = synth.make_inputs(wl, conv_bias=True)
        x, w, cb, b = (torch.from_numpy(t[k]).to(dev) for k in ("x", "w", "conv_bias", "bias"))
        out = torch.empty((128, 16, 16, 32, 32), dtype=torch.float32, device=dev)

        def call(x, out, w=w, cb=cb, b=b):
            ct.ct_convT3d_scale_pool_bias(x, w, cb, b, 0.5, 1.0, 2, 1, 1, out=out)

        def sample(t=t):
            import oracle
            n = 8
            t0 = time.perf_counter()
            oracle.convT3d_scale_pool_bias(t["x"][:n], t["w"], t["conv_bias"], t["bias"], 0.5, 1.0, 2, 1, 1)
            return time.perf_counter() - t0, n / 128.0, f"{n} of 128 batch items"

        # every weight once per pooled output and input channel: 27 products per ci
        ops.append(Op("fused3d_general", call, rotate(x, out), nbytes(x, w, cb, b, out), 2 * out.numel() * 3 * 27,
                      "hbm", HBM_PEAK_GBS, [wl.description + ", conv bias, output_padding=1"], sample))

    if "avgpool3d_nopad" in names:
        # the large pooling shape with count_include_pad=False (divisor = taps
        # inside the input), on the streaming kernel
        wl = synth.WORKLOADS["c3"]
        log(f"inputs: {wl.description}, count_include_pad=False (8.6 GB host generation)")
        xh = synth.normal(wl.seed, synth.STREAM_X, wl.x_shape)
        x = torch.from_numpy(xh).to(dev)
        out = torch.empty((16, 32, 64, 64, 128), dtype=torch.float32, device=dev)

        def call(x, out):
            ct.ct_avgpool3d(x, 3, 2, 1, False, out=out)

        def sample(xh=xh):
            import oracle
            k = 64
            t0 = time.perf_counter()
            oracle.avgpool3d(xh.reshape(512, 128, 128, 256)[:k][:, None], 3, 2, 1, False)
            return time.perf_counter() - t0, k / 512.0, f"{k} of 512 (n,c) slices"

        ops.append(Op("avgpool3d_nopad", call, rotate(x, out), nbytes(x, out), 27 * out.numel(), "hbm",
                      HBM_PEAK_GBS, [wl.description + ", count_include_pad=False"], sample))

    if "convT1d_general" in names:
        # the 1D conv shapes with stride 2, pad 1, output_padding 1 and a bias,
        # on the general gather kernel (L_out = 2L + 10)
        wl = synth.WORKLOADS["c4"]
        log(f"inputs: {wl.description}, stride 2, pad 1, output_padding 1, bias")
        t = synth.make_inputs(wl, conv_bias=True)
        x, w, bg = (torch.from_numpy(t[k]).to(dev) for k in ("x", "w", "bias"))
        out = torch.empty((32, 64, 262154), dtype=torch.float32, device=dev)

        def call(x, out, w=w, bg=bg):
            ct.ct_convT1d(x, w, bg, 2, 1, 3, 1, out=out)

        def sample(t=t):
            import oracle
            n = 4
            t0 = time.perf_counter()
            oracle.convT1d(t["x"][:n], t["w"], t["bias"], 2, 1, 3, 1)
            return time.perf_counter() - t0, n / 32.0, f"{n} of 32 batch items"

        # every input-weight product once, as at stride 1; on the fp32 matrix
        # cores (two stride-1 gathers), so bound by their peak
        flops = 2 * 32 * 32 * 131072 * 5 * 64
        ops.append(Op("convT1d_general", call, rotate(x, out), nbytes(x, w, bg, out), flops, "mfma",
                      MFMA_F32_PEAK_TFLOPS,
                      [wl.description + ", stride 2, pad 1, output_padding 1, bias"], sample))

    if "copy" in names:
        n = 1 << 28                      # 1 GiB of fp32
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)

        def call(src, dst):
            dst.copy_(src)

        ops.append(Op("copy", call, [(src, dst)], 2 * 4 * n, 0, "hbm", HBM_PEAK_GBS,
                      ["device copy 1 GiB fp32"], None))
    return ops


# ------------------------------------------------- rocprofv3 summaries --
def _csv_rows(path):
    import csv
    files = [path] if os.path.isfile(path) else [
        os.path.join(dp, f) for dp, _, fs in os.walk(path) for f in fs]
    rows = []
    for f in sorted(files):
        if f.endswith(".csv"):
            rows.extend(csv.DictReader(open(f)))
    return rows


def summarize_trace(path, ops=None):
    """Markdown table of a `rocprofv3 --kernel-trace` run: per kernel, calls
    and duration statistics in microseconds, and algorithmic GB/s at the
    average duration.  `ops`: the ops of the profiled run (see kernel_key)."""
    durs = {}
    for r in _csv_rows(path):
        if "Kernel_Name" in r and "Start_Timestamp" in r and "End_Timestamp" in r:
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            durs.setdefault(r["Kernel_Name"], []).append(d)
    total = sum(sum(v) for v in durs.values()) or 1.0
    print("| kernel | calls | avg us | min us | max us | share | algorithmic GB/s at avg |")
    print("|---|---|---|---|---|---|---|")
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        k = kernel_key(name, ops)
        avg = sum(v) / len(v)
        gbs = f"{k[2] / avg / 1e3:.0f}" if k else "-"
        short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        label = f"{k[0]} (`{short}`)" if k else f"`{short}`"
        print(f"| {label} | {len(v)} | {avg:.1f} | {min(v):.1f} | {max(v):.1f} | "
              f"{100 * sum(v) / total:.2f}% | {gbs} |")


def summarize_counters(fetch_path, write_path, dst=None, ops=None):
    """HBM bytes per launch from two `rocprofv3 --pmc` runs (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads
    for the bench's 1 GiB device copy; writes profiles/traffic.json (with a
    hash of each kernel's source) and prints a markdown table."""
    def per_kernel(path, counter):
        vals, copy = {}, []
        for r in _csv_rows(path):
            if r.get("Counter_Name") != counter:
                continue
            v = float(r["Counter_Value"])
            if "copyBuffer" in r["Kernel_Name"]:
                copy.append(v)
                continue
            k = kernel_key(r["Kernel_Name"], ops)
            if k:
                vals.setdefault(k, []).append(v)
        # the 1 GiB copy is the largest copy dispatch; the uploads of the inputs and
        # the buffer-set clones are smaller copies through the same kernel
        copy = [v for v in copy if copy and v >= 0.9 * max(copy)]
        return {k: sum(v) / len(v) for k, v in vals.items()}, (sum(copy) / len(copy) if copy else None)
    fetch, fcopy = per_kernel(fetch_path, "FETCH_SIZE")
    write, wcopy = per_kernel(write_path, "WRITE_SIZE")
    if not fcopy or not wcopy:
        raise SystemExit("no 1 GiB copy dispatch found: run the counters with --ops ...,copy")
    gib_kib = float(1 << 20)
    fs, ws = gib_kib / fcopy, gib_kib / wcopy
    out = {}
    print(f"Calibration (1 GiB copy): FETCH_SIZE {fcopy:.0f} KiB, WRITE_SIZE {wcopy:.0f} KiB per "
          f"dispatch -> scale {fs:.4f} / {ws:.4f}.\n")
    print("| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read bytes | scaled write bytes | "
          "total bytes | algorithmic bytes | total / algorithmic |")
    print("|---|---|---|---|---|---|---|---|")
    for (key, src, alg) in sorted(set(fetch) & set(write), key=lambda k: -k[2]):
        rb, wb = fetch[(key, src, alg)] * 1024 * fs, write[(key, src, alg)] * 1024 * ws
        out[key] = {"bytes_per_launch": int(rb + wb), "read_bytes": int(rb), "write_bytes": int(wb),
                    "source_sha256_16": source_hash(None, src), "source": src,
                    "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)}
        print(f"| {key} | {fetch[(key, src, alg)]:.0f} | {write[(key, src, alg)]:.0f} | {rb:.4g} | "
              f"{wb:.4g} | {rb + wb:.4g} | {alg:.4g} | {(rb + wb) / alg:.3f} |")
    dst = dst or os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(dst):                  # merge with the other runs' kernels
        try:
            prev = json.load(open(dst))
        except (OSError, ValueError):
            prev = {}
        prev.update(out)
        out = prev
    json.dump(out, open(dst, "w"), indent=1)
    print(f"\nwrote {os.path.relpath(dst, ROOT)}")


def summarize_pmc(paths, dst=None, ops=None):
    """Mean per dispatch of every counter in `rocprofv3 --pmc` runs (one or
    more output folders), per kernel of the bench, with figures derived from
    them where present: MfmaUtil (percent of SIMD cycles the matrix pipe was
    busy, rocprofv3's derived counter), VALU and SALU instructions per MFMA
    instruction, and GRBM_GUI_ACTIVE cycles per microsecond of dispatch.
    Writes profiles/counters.json (with a hash of each kernel's source) and
    prints a markdown table."""
    vals, durs = {}, {}
    for path in paths:
        for r in _csv_rows(path):
            if "Counter_Name" not in r:
                continue
            k = kernel_key(r["Kernel_Name"], ops)
            if not k:
                continue
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            durs.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(d)
    out = {}
    names = sorted({c for v in vals.values() for c in v})
    print("| kernel | " + " | ".join(names) + " | VALU / MFMA | SALU / MFMA | GRBM cycles / us |")
    print("|---|" + "---|" * (len(names) + 3))
    for (key, src, alg), cs in sorted(vals.items(), key=lambda kv: kv[0][0]):
        mean = {c: sum(v) / len(v) for c, v in cs.items()}
        rec = {"counters": mean, "source": src, "source_sha256_16": source_hash(None, src)}
        mf = mean.get("SQ_INSTS_MFMA")
        if mf:
            if "SQ_INSTS_VALU" in mean:
                rec["valu_per_mfma"] = mean["SQ_INSTS_VALU"] / mf
            if "SQ_INSTS_SALU" in mean:
                rec["salu_per_mfma"] = mean["SQ_INSTS_SALU"] / mf
        if "GRBM_GUI_ACTIVE" in mean:
            dd = durs[(key, src, alg)]["GRBM_GUI_ACTIVE"]
            rec["grbm_cycles_per_us"] = mean["GRBM_GUI_ACTIVE"] / (sum(dd) / len(dd))
        out[key + " | " + src] = rec
        cells = [f"{mean[c]:.4g}" if c in mean else "-" for c in names]
        extra = [f"{rec[f]:.3g}" if f in rec else "-" for f in
                 ("valu_per_mfma", "salu_per_mfma", "grbm_cycles_per_us")]
        print(f"| {key} (`{src}`) | " + " | ".join(cells + extra) + " |")
    dst = dst or os.path.join(ROOT, "profiles", "counters.json")
    json.dump(out, open(dst, "w"), indent=1)
    print(f"\nwrote {os.path.relpath(dst, ROOT)}")


def time_copy(torch, dev, stream, reps=20):
    """GB/s (read + write bytes) of a plain 1 GiB fp32 device copy."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return round(2 * 4 * n / ms / 1e6, 1)


def time_write(torch, dev, stream, reps=20):
    """GB/s of a write-only stream of non-constant data: 1 GiB of fp32 written
    from a 1 MiB cache-resident source broadcast over it (torch's elementwise
    copy, 16-byte stores).  The write-dominated fused ops are bound by this
    rate rather than by the copy rate; a constant fill runs faster on this
    part and is no reference for real data."""
    n = 1 << 28
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    src = torch.randn(1 << 18, generator=g, device=dev)
    dst = torch.empty((1024, 1 << 18), dtype=torch.float32, device=dev)
    view = src.expand(1024, 1 << 18)
    for _ in range(3):
        dst.copy_(view)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        dst.copy_(view)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return round(4 * n / ms / 1e6, 1)


def time_small_fused(torch, dev, stream, reps=200):
    """Per-call time of the small fused workload [2,3,8,16,16] -> [2,16,7,15,15]
    (cache-resident, launch-bound): GPU time per call from HIP events around
    `reps` back-to-back calls, and host time per call (enqueue rate, the
    same calls timed with a wall clock up to the last enqueue); isolated calls
    (synchronised around each); and calls replayed from a HIP graph."""
    import synth
    import transposed_conv_pooling_amd as ct
    wl = synth.WORKLOADS["c1"]
    t = synth.make_inputs(wl)
    x, w, bias = (torch.from_numpy(t[k]).to(dev) for k in ("x", "w", "bias"))
    out = torch.empty((2, 16, 7, 15, 15), dtype=torch.float32, device=dev)
    for _ in range(10):
        ct.ct_convT3d_scale_pool_bias(x, w, None, bias, 0.5, 1.0, out=out)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    h0 = time.perf_counter()
    for _ in range(reps):
        ct.ct_convT3d_scale_pool_bias(x, w, None, bias, 0.5, 1.0, out=out)
    h1 = time.perf_counter()
    b.record(stream)
    torch.cuda.synchronize()
    back_to_back_us = a.elapsed_time(b) * 1e3 / reps
    single = []
    for _ in range(20):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        ct.ct_convT3d_scale_pool_bias(x, w, None, bias, 0.5, 1.0, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        single.append(e0.elapsed_time(e1) * 1e3)
    # the same call captured 100 times in one HIP graph and replayed: the
    # launches then cost the host nothing, and the GPU time per call remains
    n_graph = 100
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n_graph):
            ct.ct_convT3d_scale_pool_bias(x, w, None, bias, 0.5, 1.0, out=out)
    g.replay()
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(10):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    graph_us = a.elapsed_time(b) * 1e3 / (10 * n_graph)
    alg = int(x.numel() * 4 + w.numel() * 4 + bias.numel() * 4 + out.numel() * 4)
    return {"workload": wl.description, "us_per_call_back_to_back": round(back_to_back_us, 2),
            "us_per_call_isolated": round(float(np.median(single)), 2),
            "us_per_call_graph": round(graph_us, 2),
            "host_us_per_call": round((h1 - h0) * 1e6 / reps, 2), "alg_bytes": alg}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_one_thread():
    """The oracle on one host thread: the small fused workload (mean of 10
    runs) and the full-size fp32 fused workload (one run), in ms."""
    import ctypes

    import oracle
    import synth
    gomp = ctypes.CDLL("libgomp.so.1")
    before = oracle.num_threads()
    gomp.omp_set_num_threads(1)
    try:
        res = {}
        t = synth.make_inputs(synth.WORKLOADS["c1"])
        t0 = time.perf_counter()
        for _ in range(10):
            oracle.convT3d_scale_pool_bias(t["x"], t["w"], None, t["bias"], 0.5, 1.0)
        res["fused_small_c1"] = round((time.perf_counter() - t0) * 100, 3)
        t = synth.make_inputs(synth.WORKLOADS["c2"])
        t0 = time.perf_counter()
        oracle.convT3d_scale_pool_bias(t["x"], t["w"], None, t["bias"], 0.5, 1.0)
        res["fused3d_f32_c2"] = round((time.perf_counter() - t0) * 1e3, 1)
        res["threads"] = oracle.num_threads()
    finally:
        gomp.omp_set_num_threads(before)
    return res


def _ops_opt(argv):
    """Strip an `--ops a,b` option from a summary command's arguments."""
    if "--ops" in argv:
        i = argv.index("--ops")
        return argv[:i] + argv[i + 2:], set(argv[i + 1].split(","))
    return argv, None


def main():
    if len(sys.argv) > 1 and sys.argv[1] in ("--summarize-trace", "--summarize-counters",
                                              "--summarize-pmc"):
        args, ops = _ops_opt(sys.argv[2:])
        if sys.argv[1] == "--summarize-trace":
            summarize_trace(args[0], ops)
        elif sys.argv[1] == "--summarize-counters":
            summarize_counters(args[0], args[1], ops=ops)
        else:
            summarize_pmc(args, ops=ops)
        return _report_ambiguous()
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--ops", default="fused3d_f32,avgpool3d,convT1d,fused3d_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-small", action="store_true",
                    help="skip the per-call timing of the small fused workload")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the ops shard with no exchange along batch, but only the single-GPU "
              "kernel is built and measured)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    names = [s for s in args.ops.split(",") if s]
    ops = make_ops(names, dev)
    stream = torch.cuda.current_stream(dev)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        for op in ops:
            op.run()
    torch.cuda.synchronize()

    ev = {op.name: [] for op in ops}
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_start = torch.cuda.Event(enable_timing=True)
    step_end = torch.cuda.Event(enable_timing=True)
    step_start.record(stream)
    for _ in range(args.steps):
        for op in ops:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            op.run()
            b.record(stream)
            ev[op.name].append((a, b))
    step_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    gpu_ms_per_step = step_start.elapsed_time(step_end) / args.steps

    # warm: the same op back to back on its first buffer set (the fused
    # workloads then run out of the Infinity Cache); reported beside the
    # cold, rotated figure that the step uses
    warm = {}
    for op in ops:
        if len(op.sets) == 1:
            continue
        evs = []
        for _ in range(max(args.steps, 10)):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            op.run_warm()
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        warm[op.name] = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    # a plain 1 GiB device copy: the bandwidth this machine's HBM gives a simple
    # stream, the second denominator beside the 8 TB/s peak
    copy_gbs = None
    if "copy" not in names:
        copy_gbs = time_copy(torch, dev, stream)
    write_gbs = time_write(torch, dev, stream)

    per_op = {}
    total_bytes = 0
    for op in ops:
        ms = [a.elapsed_time(b) for a, b in ev[op.name]]
        avg = float(np.mean(ms))
        d = {"ms": round(avg, 5), "ms_median": round(float(np.median(ms)), 5),
             "ms_min": round(float(np.min(ms)), 5),
             "alg_bytes": op.alg_bytes, "GB_s": round(op.alg_bytes / avg / 1e6, 1),
             "hbm_frac": round(op.alg_bytes / avg / 1e6 / HBM_PEAK_GBS, 4)}
        if copy_gbs:
            d["copy_frac"] = round(op.alg_bytes / avg / 1e6 / copy_gbs, 4)
        if op.name in warm:
            d["ms_warm"] = round(warm[op.name], 5)
        d["buffer_sets"] = len(op.sets)
        if op.flops:
            d["GFLOP_s"] = round(op.flops / avg / 1e6, 1)
        if op.bound == "mfma":
            d["mfma_frac"] = round(op.flops / avg / 1e9 / op.peak, 4)
        d["workload"] = op.inputs[0]
        per_op[op.name] = d
        if op.name != "copy":
            total_bytes += op.alg_bytes
    if "copy" in per_op:
        copy_gbs = per_op["copy"]["GB_s"]

    small = time_small_fused(torch, dev, stream) if not args.no_small else None

    dom = max(ops, key=lambda o: per_op[o.name]["ms"])
    dms = per_op[dom.name]["ms"]
    if dom.bound == "mfma":
        achieved = dom.flops / dms / 1e9            # TFLOP/s
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": dom.peak,
                "unit": "TFLOP/s", "frac": round(achieved / dom.peak, 4)}
    else:
        achieved = dom.alg_bytes / dms / 1e6        # GB/s
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": dom.peak,
                "unit": "GB/s", "frac": round(achieved / dom.peak, 4)}
    roof["kernel"] = dom.name
    roof["traffic"] = measured_traffic(dom.name) if dom.name in OP_SOURCES else None

    cpu = None
    if not args.no_cpu_baseline and all(o.oracle_sample for o in ops):
        import oracle
        log("cpu baseline: oracle on a bounded sample of each workload")
        # each op's sample is repeated until it has run for ORACLE_MIN_S, so
        # the baseline rests on ~10 s of CPU work in all
        est_s, samples = 0.0, []
        for op in ops:
            total, reps = 0.0, 0
            while total < ORACLE_MIN_S:
                secs, frac, what = op.oracle_sample()
                total += secs
                reps += 1
            est_s += total / reps / frac
            samples.append(f"{op.name}: {what}, {reps} passes in {total:.1f} s")
        cpu = {"value": round(total_bytes / est_s / 1e9, 4), "unit": "GB/s",
               "cores": oracle.num_threads(), "kind": "oracle",
               "cpu_model": cpu_model(),
               "sample": "; ".join(samples) + f"; full step extrapolated to {est_s:.1f} s",
               "one_thread_ms": oracle_one_thread()}

    value = total_bytes / (ms_per_step / 1e3) / 1e9 if total_bytes else per_op["copy"]["GB_s"]
    line = {
        "metric": "achieved HBM GB/s (and % of peak) per op; convT1d GFLOP/s; ms/call",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "gpu_ms_per_step": round(gpu_ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "+".join(dict.fromkeys(o.arith for o in ops)),
        "data": "synthetic (seeded Philox N(0,1) activations and biases, U(+-1/sqrt(fan)) weights)",
        "config": {"workload": "one full-size pass of " + ", ".join(o.name for o in ops),
                   "ops": {o.name: o.inputs[0] for o in ops}},
        "ops": per_op,
        "roofline": roof,
        "copy_GB_s": copy_gbs,
        "write_GB_s": write_gbs,
        "small_fused_c1": small,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
