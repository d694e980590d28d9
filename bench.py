"""Benchmark of the exact attention forward on one MI355X.

One step = one forward pass over the whole batch of the workload (one
``attn_fwd`` launch; the partial-attention and merge launches of a key-range
split; or the block quantisation of Q, K and V followed by the block-scaled
e4m3 attention of the fp8 input pipeline), inputs resident in HBM.  Prints ONE
JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

The untimed warm-up lasts at least --warmup steps and at least about 1.5 s
of back-to-back work (the given count is a minimum): a GPU coming out of idle
first runs below, then above, the clock it settles at under sustained load,
and the timed steps should see the settled clock (the ZYFA article, "What the
numbers establish, and where they overstate", makes the same point about
sustained clocks).  Exactly --steps steps are timed (without --steps: about
1 s of work).  The shader clock and the socket power are sampled through
amdsmi during the last part of the warm-up and the timed loop; the JSON line
reports them, the percentage of the peak normalised to the clock, and the
median, best, first and last per-launch times.

Throughput is matmul TFLOP/s: 4 * B * Hq * D * (visible query/key pairs) per
step (the QK^T and PV products; softmax work is not counted).  The roofline
object prices the same flops against the dense MFMA peak of the compute dtype,
using the attention kernel's own average duration from HIP events recorded
on the launch stream around that launch (around the whole step for a key-range
split, whose merge launch is then counted too).  The cpu_baseline object times the fp64 oracle on a bounded
sample of the same workload on the host cores.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

from exact_io_aware_attn_amd import attn as A
from exact_io_aware_attn_amd.inputs import WORKLOADS, make_grad, make_inputs

METRIC = "attention fwd TFLOPS on 1 MI355X and % of dense bf16/fp8 MFMA peak"
# the backward workload counts the five matrix products of the gradients
# (recomputed Q K^T, dO V^T, P^T dO, dS K, dS^T Q): 2.5x the forward's flops
METRIC_BWD = "attention bwd TFLOPS on 1 MI355X (5 matmuls counted) and % of dense bf16 MFMA peak"
# MI355X dense MFMA peaks (TFLOP/s): bf16 2.5 PF, fp8 5.0 PF, fp32 157.3 TF.
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
# the gated configuration: GQA causal prefill, B2 Hq32 Hkv8 N8192 D128, bf16
DEFAULT_WORKLOAD = "gqa_causal_bf16"
# datasheet clock of the dense peaks above (MHz)
PEAK_SCLK_MHZ = 2400.0
# The pages' MI355X figure closest to a workload (TFLOP/s), reported as
# context only: the ZYFA article, "What the numbers establish, and where they
# overstate", gives 2672 TFLOP/s for its own fp8 kernel on causal prefill at
# 32K tokens, D = 128, Gaussian inputs, with an unstated head count.
CONTEXT_TFLOPS = {"fp8_p8_causal_32k": 2672.0, "fp8_lean_causal_32k": 2672.0}
INPUTS = {
    "fp8": "i.i.d. N(0,1), 1% outlier channels x8, per-tensor e4m3, seed 0",
    "fp8blk": "bf16 i.i.d. N(0,1), 1% outlier channels x8 shared by Q and K, seed 0; "
              "quantised on the device, one descale per 64 rows, Q and K Hadamard-rotated",
}


# HBM bytes per launch measured with rocprofv3 (FETCH_SIZE and WRITE_SIZE per
# dispatch, scaled by what the same counters read for a plain device copy of
# known size: reads x2.00, writes x1.00), for the dominant kernel of a
# workload.  Each entry is tied to a hash of the sources of that kernel;
# when they have changed since the counters were taken, traffic is null.
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "exact_io_aware_attn_amd", "csrc")
# sources of the direct-to-LDS and e4m3-probability kernels (the launch
# rules, causal tile pairing included, live in attn_launch.h)
_PIPE = ("attn_common.h", "attn_dma.h", "attn_launch.h", "attn_fwd_pipe.hip")
# sources of the bf16 kernel of head dims 64 and 128
_BF16 = ("attn_common.h", "attn_dma.h", "attn_launch.h", "attn_fwd_bf16.hip")
_P8 = ("attn_common.h", "attn_dma.h", "attn_launch.h", "attn_fwd_p8.hip")
# the split-D kernels: four waves (D up to 960) and eight (D = 1024)
_SPLITD = ("attn_common.h", "attn_dma.h", "attn_launch.h", "attn_fwd_splitd.hip")
_SPLITD8 = ("attn_common.h", "attn_dma.h", "attn_launch.h", "attn_fwd_splitd8.hip")
# the wide-head kernel (bf16 D = 192..512)
_WIDE = ("attn_common.h", "attn_dma.h", "attn_launch.h", "attn_fwd_wide.hip")
# the backward's three launches
_BWD = ("attn_common.h", "attn_dma.h", "attn_launch.h", "attn_bwd.h", "attn_bwd.hip")
MEASURED_TRAFFIC = {
    # workload: (kernel sources, source hash, bytes read, bytes written)
    "prefill_causal_bf16": (_BF16, "233822d0f6f3ebb5", 281102.375 * 2 * 1024, 137414.96875 * 1024),
    "gqa_causal_bf16": (_BF16, "233822d0f6f3ebb5", 144185.4375 * 2 * 1024, 133120.0 * 1024),
    "gqa_cross_bf16": (_BF16, "233822d0f6f3ebb5", 49249.25 * 2 * 1024, 33280.0 * 1024),
    "fp8_outlier": (_PIPE, "b33c0f454fba9573", 122953.5 * 2 * 1024, 99840.0 * 1024),
    # the attention launch of the fp8 input pipeline (the quantisers read and
    # write each byte once)
    "fp8_blocks_outlier": (_PIPE, "b33c0f454fba9573", 123004.5 * 2 * 1024, 99840.0 * 1024),
    "splitd_bf16_d1024": (_SPLITD8, "dca91d739d485894", 163938.5 * 2 * 1024, 68142.9375 * 1024),
    "splitd_bf16_d768": (_SPLITD, "5de55f883bc0be40", 123050.0 * 2 * 1024, 49280.0 * 1024),
    "splitd_bf16_d512": (_WIDE, "f6d4df4d3cdd1c55", 49594.5 * 2 * 1024, 33408.0 * 1024),
    # the partial-attention launch over 8 key ranges (the merge launch after
    # it reads and writes its parts once)
    "chunk_prefill_splitkv_bf16": (_BF16, "233822d0f6f3ebb5", 73820.5625 * 2 * 1024, 33088.25 * 1024),
    # the whole backward step: prep + dK/dV + dQ launches
    "bwd_causal_bf16": (_BWD, "6e982fcd75cec507", 678817.5 * 2 * 1024, 397390.265625 * 1024),
    "bwd_causal_bf16_d256": (_BWD, "6e982fcd75cec507", 692962.03125 * 2 * 1024, 396023.0625 * 1024),
    "bwd_causal_bf16_d512": (_BWD, "6e982fcd75cec507", 1000050.78125 * 2 * 1024, 446495.171875 * 1024),
    "prefill_causal_bf16_poly": (_PIPE, "b33c0f454fba9573", 262696.03125 * 2 * 1024, 133120.0 * 1024),
    "fp8_p8_outlier": (_P8, "40c93540ee3a0f74", 169015.1875 * 2 * 1024, 99840.0 * 1024),
    "fp8_lean_outlier": (_P8, "40c93540ee3a0f74", 122964.25 * 2 * 1024, 99840.0 * 1024),
    "fp8_lean_causal_32k": (_P8, "40c93540ee3a0f74", 440425.3125 * 2 * 1024, 266244.296875 * 1024),
}


def measured_traffic(name):
    """HBM bytes per launch for the workload, or None if unmeasured or stale."""
    entry = MEASURED_TRAFFIC.get(name)
    if entry is None:
        return None
    files, digest, rd, wr = entry
    m = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            m.update(fh.read())
    return int(round(rd + wr)) if m.hexdigest()[:16] == digest else None


class ClockSampler:
    """Samples the GPU's current shader (gfx) clock and socket power in a
    background thread through amdsmi, every `period` seconds, between start()
    and stop().  Reports nothing (None) where amdsmi or the metric is
    unavailable."""

    def __init__(self, period=0.01, enabled=True):
        import threading
        self.period = period
        self.samples = []
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        self._handle = None
        self._smi = None
        if not enabled:
            self.error = "not sampled (--no-sclk)"
            return
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            self._handle = handles[0] if handles else None
            self._smi = amdsmi
        except Exception as e:  # pragma: no cover - depends on the machine
            self.error = f"amdsmi unavailable: {type(e).__name__}"

    def _read(self):
        """(gfx clock in MHz or None, socket power in W or None)."""
        smi = self._smi
        try:
            m = smi.amdsmi_get_gpu_metrics_info(self._handle)
            pw = m.get("current_socket_power")
            pw = float(pw) if isinstance(pw, (int, float)) and 0 < pw < 5000 else None
            clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 10000]
            if clks:
                return float(np.mean(clks)), pw  # the XCDs' clocks (all busy under these kernels)
            c = m.get("current_gfxclk")
            if isinstance(c, (int, float)) and 0 < c < 10000:
                return float(c), pw
        except Exception:
            pass
        info = smi.amdsmi_get_clock_info(self._handle, smi.AmdSmiClkType.GFX)
        c = info.get("clk")
        return (float(c) if isinstance(c, (int, float)) and 0 < c < 10000 else None), None

    def _run(self):
        while not self._stop.is_set():
            try:
                c, pw = self._read()
                if c is not None:
                    self.samples.append((time.perf_counter(), c, pw))
            except Exception as e:  # pragma: no cover
                self.error = f"amdsmi read failed: {type(e).__name__}"
                return
            self._stop.wait(self.period)

    def start(self):
        import threading
        if self._smi is None or self._handle is None:
            return
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        if self._smi is not None:
            try:
                self._smi.amdsmi_shut_down()
            except Exception:  # pragma: no cover
                pass

    def summary(self, t0=None, t1=None):
        """Median, min and max of the samples taken between t0 and t1
        (perf_counter seconds: the timed loop), or of all of them if none
        falls there.  Samples taken while the GPU idles between the warm-up
        and the timed loop read the idle clock, hence the window."""
        if not self.samples:
            return None
        t = np.asarray([a for a, _, _ in self.samples])
        c = np.asarray([b for _, b, _ in self.samples])
        pw = np.asarray([np.nan if x is None else x for _, _, x in self.samples], dtype=np.float64)
        inside = (t >= t0) & (t <= t1) if t0 is not None and t1 is not None else np.ones(len(c), bool)
        window = "the timed loop"
        if not inside.any():
            inside, window = np.ones(len(c), bool), "the last 0.5 s of warm-up and the timed loop"
        s = c[inside]
        p = pw[inside]
        p = p[np.isfinite(p)]
        return {"median_mhz": round(float(np.median(s)), 1), "min_mhz": round(float(s.min()), 1),
                "max_mhz": round(float(s.max()), 1), "samples": int(s.size),
                "socket_power_w": round(float(np.median(p)), 1) if p.size else None,
                "source": f"amdsmi current gfx clock (mean over XCDs) and socket power, sampled every 10 ms, "
                          f"over {window}"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: about 1 s of work)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="minimum untimed steps (the warm-up also lasts at least about 1.5 s)")
    ap.add_argument("--warmup-seconds", type=float, default=1.5,
                    help="minimum duration of the warm-up (0 for counter-collection runs)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sclk", action="store_true", help="do not sample the shader clock (profiler runs)")
    ap.add_argument("--cpu-heads", type=int, default=0, help="heads in the oracle sample (0 = time budget)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="time budget of the oracle sample")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of attention, run a plain device copy of this many MiB (HBM counter calibration)")
    return ap.parse_args()


def copy_calibration(mib, steps):
    """Plain device-to-device copy of a known size: the bytes the HBM traffic
    counters should report per launch are exactly 2 x mib MiB (read + write)."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_launch": n * 4, "bytes_written_per_launch": n * 4,
                                           "launches": steps}}), flush=True)


def is_bwd(w):
    return w.extra.get("pass") == "bwd"


def step_flops(w):
    return float(w.flops) * (2.5 if is_bwd(w) else 1.0)


def gpu_inputs(w, dev):
    inp = make_inputs(w)
    if is_bwd(w):
        inp = (*inp, make_grad(w))
    if w.dtype == "fp8blk":
        return tuple(t.to(dev) for t in inp), inp
    if w.dtype == "fp8":
        q8, k8, v8, desc = inp
        ds = [torch.tensor([float(x)], dtype=torch.float32, device=dev) for x in desc]
        return (q8.to(dev), k8.to(dev), v8.to(dev), *ds), inp
    return tuple(t.to(dev) for t in inp), inp


def make_step(w, dev_inp, out, lse):
    """A callable running one step; called with a pair of events it records
    them around the step's dominant kernel on the launch stream."""
    stream = torch.cuda.current_stream()

    def bracket(fn):
        def step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            fn()
            if ev is not None:
                ev[1].record(stream)
        return step

    if is_bwd(w):
        # the forward outputs once, outside the timed steps; then dQ, dK, dV
        # into buffers allocated once, with a workspace allocated once
        q, k, v, g = dev_inp
        A.fwd(q, k, v, causal=w.causal, scale=w.scale, out=out, lse=lse)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(A.bwd_workspace_bytes(w.B, w.Hq, w.Nq), dtype=torch.uint8, device=q.device)
        return bracket(lambda: A.bwd(q, k, v, out, lse, g, causal=w.causal, scale=w.scale, workspace=ws,
                                     dq=dq, dk=dk, dv=dv))
    if w.dtype == "fp8blk":
        # the fp8 input pipeline: Q and K rotated and block-quantised, V
        # block-quantised, then block-scaled e4m3 attention; buffers once
        q, k, v, signs = dev_inp
        bufs = []
        for t in (q, k, v):
            nb = (t.shape[2] + 63) // 64
            bufs.append((torch.empty(t.shape, dtype=torch.float8_e4m3fn, device=t.device),
                         torch.empty((t.shape[0], t.shape[1], nb), dtype=torch.float32, device=t.device)))
        (cq, dq), (ck, dk), (cv, dv) = bufs

        def step(ev=None):
            A.quantize_fp8(q, signs, codes=cq, descales=dq)
            A.quantize_fp8(k, signs, codes=ck, descales=dk)
            A.quantize_fp8(v, None, codes=cv, descales=dv)
            if ev is not None:
                ev[0].record(stream)
            A.fwd_fp8_blocks(cq, ck, cv, dq, dk, dv, causal=w.causal, scale=w.scale, out=out, lse=lse)
            if ev is not None:
                ev[1].record(stream)
        return step
    if w.extra.get("n_splits"):
        # key-range split: one launch over all ranges, then the LSE merge,
        # through attn_fwd_splitkv with a workspace allocated once, here
        ns = int(w.extra["n_splits"])
        q, k, v = dev_inp[:3]
        desc = tuple(dev_inp[3:]) if w.dtype == "fp8" else None
        ws = torch.empty(A.splitkv_workspace_bytes(w.B, w.Hq, w.Nq, w.D, ns), dtype=torch.uint8, device=q.device)

        return bracket(lambda: A.fwd_splitkv(q, k, v, ns, causal=w.causal, scale=w.scale, descales=desc,
                                             workspace=ws, out=out, lse=lse))
    if w.dtype == "fp8" and w.extra.get("p"):
        q, k, v, dq, dk, dv = dev_inp
        lean = w.extra["p"] == "lean"
        return bracket(lambda: A.fwd_fp8_p(q, k, v, dq, dk, dv, causal=w.causal, scale=w.scale, lean=lean, out=out,
                                           lse=lse))
    if w.dtype == "fp8":
        q, k, v, dq, dk, dv = dev_inp
        return bracket(lambda: A.fwd_fp8(q, k, v, dq, dk, dv, causal=w.causal, scale=w.scale, out=out, lse=lse))
    q, k, v = dev_inp
    if w.extra.get("exp") == "poly":
        return bracket(lambda: A.fwd_exp_poly(q, k, v, causal=w.causal, scale=w.scale, out=out, lse=lse))
    return bracket(lambda: A.fwd(q, k, v, causal=w.causal, scale=w.scale, out=out, lse=lse))


def cpu_baseline(w, host_inp, n_heads, seconds):
    """Time the fp64 oracle on (batch, head) slices of the workload: n_heads of
    them, or (n_heads == 0) as many as fit in about `seconds` (at least one)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    G = w.Hq // w.Hkv
    rng = np.random.default_rng(1)
    # distinct (batch, head) slices in random order, until the budget or the
    # whole workload is done
    order = [(int(x // w.Hq), int(x % w.Hq)) for x in rng.permutation(w.B * w.Hq)]
    if w.dtype == "fp8blk":
        q, k, v, signs = host_inp
        s = signs.numpy()

        def blk(t, b, h, sg):
            # blocks never span heads: one head's slab quantises alone exactly
            x = t[b:b + 1, h:h + 1].to(torch.float64).numpy()
            return oracle.dequantize_blocks(*oracle.quantize_blocks(x, sg))[0, 0]
        get_q = lambda b, h: blk(q, b, h, s)
        get_k = lambda b, h: blk(k, b, h, s)
        get_v = lambda b, h: blk(v, b, h, None)
    elif w.dtype == "fp8":
        q8, k8, v8, desc = host_inp

        def head(t, d, b, h):
            return oracle.e4m3fn_decode(t[b, h].view(torch.uint8).numpy()) * np.float64(d)
        get_q = lambda b, h: head(q8, desc[0], b, h)
        get_k = lambda b, h: head(k8, desc[1], b, h)
        get_v = lambda b, h: head(v8, desc[2], b, h)
    else:
        q, k, v = host_inp[:3]
        get_q = lambda b, h: q[b, h].to(torch.float64).numpy()
        get_k = lambda b, h: k[b, h].to(torch.float64).numpy()
        get_v = lambda b, h: v[b, h].to(torch.float64).numpy()
    done = 0
    t0 = time.perf_counter()
    for b, hq in order:
        if w.dtype == "fp8" and w.extra.get("p"):
            oracle.fp8p_attention_head(get_q(b, hq), get_k(b, hq // G), get_v(b, hq // G), w.scale, w.causal,
                                       lean=w.extra["p"] == "lean")
        elif is_bwd(w):
            g = host_inp[3][b, hq].to(torch.float64).numpy()
            oracle.attention_backward_head(get_q(b, hq), get_k(b, hq // G), get_v(b, hq // G), g, w.scale,
                                           w.causal)
        else:
            oracle.attention_head(get_q(b, hq), get_k(b, hq // G), get_v(b, hq // G), w.scale, w.causal)
        done += 1
        dt = time.perf_counter() - t0
        if (n_heads and done >= n_heads) or (not n_heads and dt >= seconds):
            break
    dt = time.perf_counter() - t0
    flops = 4.0 * w.D * w.visible_pairs * done * (2.5 if is_bwd(w) else 1.0)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} of {w.B * w.Hq} (batch, head) slices of {w.name} (drawn at random, seed 1), fp64 numpy, "
                  f"S materialised per head; {dt:.1f} s wall, scaled by the same flop formula",
        "cpu_model": cpu_model(),
        "os_cpu_count": os.cpu_count(),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(3)
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib, args.steps or 200)
        return
    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    A.lib()  # fail loudly if the HIP library is missing
    dev_inp, host_inp = gpu_inputs(w, dev)
    out_dtype = torch.float32 if w.dtype == "f32" else torch.bfloat16
    out = torch.empty((w.B, w.Hq, w.Nq, w.D), dtype=out_dtype, device=dev)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
    step = make_step(w, dev_inp, out, lse)

    # size the warm-up and the timed loop from a short probe (its steps count
    # as warm-up steps)
    probe = 10 if args.warmup is None else max(1, min(10, args.warmup))
    torch.cuda.synchronize()
    t_probe = time.perf_counter()
    for _ in range(probe):
        step()
    torch.cuda.synchronize()
    est = max((time.perf_counter() - t_probe) / probe, 1e-6)
    floor = int(min(20000, max(50, math.ceil(args.warmup_seconds / est)))) if args.warmup_seconds > 0 else 0
    warmup = max(args.warmup or 0, floor, probe)
    if args.steps is None:
        args.steps = int(min(5000, max(200, math.ceil(1.0 / est))))
    # the clock is sampled over the last ~0.5 s of the warm-up and the timed loop
    tail = max(0, min(warmup - probe, int(math.ceil(0.5 / est))))
    for _ in range(max(0, warmup - probe - tail)):
        step()
    clock = ClockSampler(enabled=not args.no_sclk)
    clock.start()
    for _ in range(max(0, tail)):
        step()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for pair in ev:
        step(pair)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock.stop()
    kernel_ms = np.asarray([s.elapsed_time(e) for s, e in ev])
    avg_kernel_s = float(np.mean(kernel_ms)) / 1e3

    ms_per_step = wall * 1e3 / args.steps
    flops = step_flops(w)
    value = flops / (wall / args.steps) / 1e12
    achieved = flops / avg_kernel_s / 1e12
    compute_dtype = "fp8" if w.dtype == "fp8blk" else w.dtype
    peak = PEAK_TFLOPS[compute_dtype]
    sclk = clock.summary(t0, t0 + wall)
    res = {
        "metric": METRIC_BWD if is_bwd(w) else METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": compute_dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nkv": w.Nkv, "D": w.D,
            "causal": w.causal, "scale": "1/sqrt(D)", "inputs": INPUTS.get(w.dtype, "i.i.d. N(0,1), seed 0"),
            **({"exponential": "cubic polynomial on the FMA pipe (relative error <= 8.6e-5)"}
               if w.extra.get("exp") == "poly" else {}),
            **({"probabilities": "e4m3, one power-of-two scale per 64-key block, " +
                                 ("Lean P codes" if w.extra["p"] == "lean" else "exact codes") +
                                 "; P V and the row sum on the fp8 matrix instruction"}
               if w.extra.get("p") else {}),
            **({"timed": "attn_bwd: delta/lse2 prep + dK/dV + dQ launches (forward outputs computed once, "
                         "before the timed steps); roofline over the whole backward"} if is_bwd(w) else {}),
            **({"timed": "block quantisation of Q, K (rotated) and V + block-scaled e4m3 attention; "
                         "roofline on the attention launch alone"} if w.dtype == "fp8blk" else {}),
            **({"n_splits": int(w.extra["n_splits"]),
                "timed": "partial-attention launch over all key ranges + LSE merge launch"}
               if w.extra.get("n_splits") else {}),
            "flops_per_step": flops,
            "pct_of_dense_peak": round(100.0 * value / peak, 2),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(w.name),
            "frac_at_measured_sclk": (round(achieved / (peak * sclk["median_mhz"] / PEAK_SCLK_MHZ), 4)
                                      if sclk else None),
        },
        "sclk": sclk if sclk else {"median_mhz": None, "note": clock.error or "no samples"},
        "kernel_ms": {
            "mean": round(float(kernel_ms.mean()), 5),
            "median": round(float(np.median(kernel_ms)), 5),
            "min": round(float(kernel_ms.min()), 5),
            "first": round(float(kernel_ms[0]), 5),
            "last": round(float(kernel_ms[-1]), 5),
            "what": "HIP events on the launch stream around the dominant kernel of each timed step",
        },
        "context_tflops": ({"value": CONTEXT_TFLOPS[w.name], "source": "ZYFA article, own fp8 kernel, other "
                           "head count: context, not a baseline"} if w.name in CONTEXT_TFLOPS else None),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, host_inp, args.cpu_heads, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
