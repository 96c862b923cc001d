#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet hot path on one MI355X.

One step = one gdn_chunk_fwd over the prefill workload (default: the 262,144-token native
context, B=1, 16 heads, dk=dv=128, chunk 64, bf16 inputs, long-memory gates, fp32 output and
state) followed by the decode workload: 64 consecutive gdn_decode_step calls (B=256 sequences,
32 heads, dk=dv=128, fp32 state [256,32,128,128] updated in place, one pre-drawn token per
call).  Inputs are seeded synthetic tensors with the recipe's distributions (gdn_inputs.py;
the long prefill's are drawn on the GPU with torch's generator), resident in HBM before the
timed region.

Prints ONE JSON line:  value = prefill tokens/s (B*T / mean prefill launch time), with the
decode state GB/s, both kernels' rooflines (algorithmic bytes / measured launch time,
against 8 TB/s HBM and 2.5 PFLOP/s dense fp16/bf16 MFMA), and the fp64 oracle's throughput
on the host cores as a reported CPU baseline.  Outside the step, "decode_tokens" reports
gdn_decode_tokens over T = 2, 4, 8 tokens of the decode workload per call (one read and one
write of every state per call; in place, and for T = 8 also into a separate output state, as a
verifier keeping the old state would call it); "prologue_and_packed" reports the prefill with
the fused input prologue and a packed batch of 32 variable-length sequences, and the backward,
all on the 4096-token workload; "qsa_indexer" reports the QSA compressed indexer
(gdn_qsa_index) on a 65536-token sequence; "prefill_other_workloads" times the other prefill
workloads (B=1 T=4096 H=16; B=8 T=8192 with grouped heads); "prefill_plans_compared" times
the step's prefill workload under each chunk-parallel plan that takes it (split: per-chunk
records through a workspace; segmented: segments of each chain in parallel, chained through
their affine state maps); "decode_cycled_states" times the
decode step over four separate state buffers in turn, so that no state is still in the
last-level cache when it is read again; "measured_peaks" reports what a plain device copy and a
dense bf16 matrix product reach in the same run.
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA, vendor figure
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma.json")
KERNEL_SOURCES = {
    # the split plan (prep + scan), the fused kernel and decode, each with the shared header
    "prefill": [os.path.join(ROOT, "linear_attention_token_gdn_amd", "csrc", n)
                for n in ("chunk_split.hip", "gdn_internal.h")],
    "fused": [os.path.join(ROOT, "linear_attention_token_gdn_amd", "csrc", n)
              for n in ("chunk_mfma.hip", "gdn_internal.h")],
    "segmented": [os.path.join(ROOT, "linear_attention_token_gdn_amd", "csrc", n)
                  for n in ("chunk_mfma.hip", "gdn_internal.h")],
    "decode": [os.path.join(ROOT, "linear_attention_token_gdn_amd", "csrc", n)
               for n in ("decode.hip", "gdn_internal.h")],
}


# ------------------------------------------------------------------ algorithmic counts
def prefill_flops(B, T, Hk, Hv, dk, dv, C):
    """Algorithmic FLOPs of the chunk-parallel form: only the needed triangles, KK^T and QK^T
    once per q/k head; multiply-add = 2."""
    total = 0
    for t0 in range(0, T, C):
        L = min(C, T - t0)
        qk = 2 * L * L * dk                                   # lower KK^T (strict) + QK^T (incl)
        v = ((L ** 3 - L) // 3 + L * (L - 1) * (dk + dv)       # inverse, U, W
             + L * (L + 1) * dv + 6 * L * dk * dv)             # P Delta, W S, Q S, K^T Delta
        total += Hk * qk + Hv * v
    return B * total


def prefill_bytes(B, T, Hk, Hv, dk, dv, in_bytes=2, out_bytes=4, has_s0=False):
    rd = B * T * (2 * Hk * dk + Hv * dv + 2 * Hv) * in_bytes
    if has_s0:
        rd += B * Hv * dk * dv * 4
    wr = B * T * Hv * dv * out_bytes + B * Hv * dk * dv * 4
    return rd + wr


def decode_bytes(B, Hk, Hv, dk, dv, T=1, in_bytes=2, out_bytes=4):
    """Algorithmic bytes of one decode call over T tokens: the state read and written once,
    plus every token's inputs and outputs."""
    state = 2 * B * Hv * dk * dv * 4
    other = B * T * ((2 * Hk * dk + Hv * dv + 2 * Hv) * in_bytes + Hv * dv * out_bytes)
    return state, state + other


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per call (the prefill's launches together; one launch for the decode) from the
    committed rocprofv3 --pmc summary, or None when absent, taken on another workload or on a
    different version of the kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    if rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_call", rec.get("bytes_per_launch"))


def measured_mfma(label, sources):
    """Matrix-core busy fraction and issued/algorithmic MFMA flops of one prefill workload from
    the committed counter summary, or None when absent or taken on other kernel sources."""
    try:
        with open(MFMA_FILE) as fh:
            rec = json.load(fh).get(label, {}).get("prefill")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[sources]):
        return None
    return {"mfma_busy_pct": round(rec["mfma_busy_pct_weighted"], 2),
            "mfma_flops_issued_over_algorithmic": round(rec["issued_over_algorithmic"], 3)}


# ------------------------------------------------------------------ CPU baseline (oracle)
def cpu_baseline(pre_inp, dec_inp, full_T, min_s=10.0):
    """The fp64 oracle on the host cores: `pre_inp` is the prefill workload's first tokens (all
    of its chains, drawn by the recipe), run repeatedly for at least `min_s` seconds; tokens/s
    is per token of the whole sequence, the same unit as the GPU figure.  Plus one decode step
    of the decode workload."""
    import numpy as np
    import oracle
    threads = min(16, len(os.sched_getaffinity(0)))
    B, T, Hk, Hv = pre_inp.q.shape[0], pre_inp.q.shape[1], pre_inp.q.shape[2], pre_inp.v.shape[2]
    reps, t = 0, time.perf_counter()
    while True:  # repeat the sample until min_s seconds of CPU time are taken
        oracle.run(pre_inp.q, pre_inp.k, pre_inp.v, pre_inp.beta, pre_inp.g, s0=pre_inp.s0,
                   nthreads=threads, want_state=True)
        reps += 1
        if time.perf_counter() - t >= min_s or reps >= 50:
            break
    pre_s = (time.perf_counter() - t) / reps
    # decode: one step of the decode workload (all 8192 states, fp64)
    st = dec_inp.s0.astype(np.float64)
    t = time.perf_counter()
    oracle.decode_step(dec_inp.q[:, 0], dec_inp.k[:, 0], dec_inp.v[:, 0], dec_inp.beta[:, 0],
                       dec_inp.g[:, 0], st, nthreads=threads)
    dec_s = time.perf_counter() - t
    Bd, Hvd, dk, dv = dec_inp.s0.shape
    state_bytes_f32 = 2 * Bd * Hvd * dk * dv * 4
    return {
        "value": B * T / pre_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
        "host_cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
        "sample": ("the first %d of the prefill workload's %d tokens, all %d chains (B=%d, %d "
                   "heads; fp64 token-by-token recurrence, chains in parallel on %d threads), "
                   "mean of %d runs: %.3f s each; plus one decode step of the decode workload in "
                   "%.3f s" % (T, full_T, B * Hv, B, Hv, threads, reps, pre_s, dec_s)),
        "decode_state_GBps_fp32_equiv": state_bytes_f32 / dec_s / 1e9,
        "cpu_model": _cpu_model(),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------ timing events
class HipEvent:
    """A HIP timing event recorded on a given stream, created with hipEventDisableSystemFence:
    recording it issues no system-scope fence, so the cache writeback and invalidation such a
    fence costs are not added to (or imposed on) the work being timed.  Same interface as
    torch.cuda.Event for what this script uses: record(stream), elapsed_time(other) in ms."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if HipEvent._hip is None:
            HipEvent._hip = ctypes.CDLL("libamdhip64.so")
        self._ct = ctypes
        self._e = ctypes.c_void_p()
        rc = HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self._e),
                                                   ctypes.c_uint(self.DISABLE_SYSTEM_FENCE))
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed (%d)" % rc)

    def record(self, stream):
        rc = HipEvent._hip.hipEventRecord(self._e, self._ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed (%d)" % rc)

    def elapsed_time(self, other):
        ms = self._ct.c_float()
        rc = HipEvent._hip.hipEventElapsedTime(self._ct.byref(ms), self._e, other._e)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return ms.value

    def __del__(self):
        if HipEvent._hip is not None and self._e:
            HipEvent._hip.hipEventDestroy(self._e)


# ------------------------------------------------------------------ the other prefill workloads
def gpu_inputs(torch, dev, idx):
    """A prefill workload's inputs drawn on the GPU with the recipe's distributions (q, k ~
    N(0,1) then L2-normalised per head, v ~ N(0,1), beta = sigmoid(N(0,1)), log alpha =
    -U(lo, hi), S0 ~ N(0, std^2)), rounded to bf16; seed 1000 + workload index."""
    from gdn_inputs import CONFIGS
    c = CONFIGS[idx]
    B, T, Hk, Hv, dk, dv = (c[k_] for k_ in ("B", "T", "Hk", "Hv", "dk", "dv"))
    g = torch.Generator(device=dev)
    g.manual_seed(1000 + idx)
    nrm = torch.nn.functional.normalize
    q = nrm(torch.randn(B, T, Hk, dk, device=dev, generator=g), dim=-1).to(torch.bfloat16)
    k = nrm(torch.randn(B, T, Hk, dk, device=dev, generator=g), dim=-1).to(torch.bfloat16)
    v = torch.randn(B, T, Hv, dv, device=dev, generator=g).to(torch.bfloat16)
    beta = torch.sigmoid(torch.randn(B, T, Hv, device=dev, generator=g)).to(torch.bfloat16)
    lo, hi = c["g_range"]
    gg = (-(torch.rand(B, T, Hv, device=dev, generator=g) * (hi - lo) + lo)).to(torch.bfloat16)
    s0 = None if c["s0_std"] is None else \
        torch.randn(B, Hv, dk, dv, device=dev, generator=g) * c["s0_std"]
    return {"q": q, "k": k, "v": v, "beta": beta, "g": gg, "s0": s0}


def prefill_configs(gdn, torch, dev, stream, names=(1, 2)):
    """The other prefill workloads (by default 1: 4,096 tokens, 16 heads; 2: 8 x 8192 tokens,
    16 q/k and 32 v heads, initial state): one call each, median of 3, with 1 GiB written
    between calls so that nothing stays in the last-level cache.  Timing inputs are drawn on
    the GPU (gpu_inputs); parity is tested on the recipe's own seeded draws."""
    from gdn_inputs import CONFIGS
    out = {}
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    for idx in names:
        c = CONFIGS[idx]
        B, T, Hk, Hv, dk, dv, C = (c[k_] for k_ in ("B", "T", "Hk", "Hv", "dk", "dv", "chunk"))
        x = gpu_inputs(torch, dev, idx)
        q, k, v, beta, gg, s0 = (x[n] for n in ("q", "k", "v", "beta", "g", "s0"))
        o = torch.empty(B, T, Hv, dv, dtype=torch.float32, device=dev)
        fs = torch.empty(B, Hv, dk, dv, dtype=torch.float32, device=dev)
        call = lambda: gdn.chunk_fwd(q, k, v, beta, gg, initial_state=s0, chunk=C, o=o,
                                     final_state=fs)
        call()
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            flush.fill_(1.0)
            e0, e1 = HipEvent(), HipEvent()
            e0.record(stream)
            call()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[1]
        fl = prefill_flops(B, T, Hk, Hv, dk, dv, C)
        by = prefill_bytes(B, T, Hk, Hv, dk, dv, has_s0=s0 is not None)
        plan = gdn.gdn_chunk_fwd_plan(B, T, Hk, Hv, dk, dv, C, gdn.GDN_BF16)
        out[c["name"]] = {
            "plan": plan,
            "ms": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "TFLOPs": round(fl / (ms * 1e-3) / 1e12, 2),
            "frac_bf16_mfma_peak": round(fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "GBps": round(by / (ms * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "frac_binding_roofline": round(max(by / (HBM_PEAK_GBS * 1e9),
                                               fl / (MFMA_BF16_PEAK_TFLOPS * 1e12)) / (ms * 1e-3), 4),
            "algorithmic_flops": fl, "algorithmic_bytes": by,
            "mfma_counters": measured_mfma("workload%d_%s" % (idx, plan),
                                           {"split": "prefill"}.get(plan, plan))}
        del q, k, v, beta, gg, s0, o, fs, x
        torch.cuda.synchronize()
    del flush
    return out


def prefill_plans(gdn, torch, dev, stream, idx,
                  plans=("split", "segmented", "segmented_formed")):
    """One prefill workload under each chunk-parallel plan that takes it (GDN_FORCE_VARIANT),
    one call each, median of 3, 1 GiB written between calls; inputs as gpu_inputs.
    "segmented_formed" is the segmented plan with GDN_SEG_NO_TM set: both of its passes form
    every chunk's (I + A)^-1 instead of the output pass reading the transition pass's."""
    from gdn_inputs import CONFIGS
    c = CONFIGS[idx]
    B, T, Hk, Hv, dk, dv, C = (c[k_] for k_ in ("B", "T", "Hk", "Hv", "dk", "dv", "chunk"))
    x = gpu_inputs(torch, dev, idx)
    o = torch.empty(B, T, Hv, dv, dtype=torch.float32, device=dev)
    fs = torch.empty(B, Hv, dk, dv, dtype=torch.float32, device=dev)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    out = {}
    old = os.environ.get("GDN_FORCE_VARIANT")
    try:
        for plan in plans:
            base = plan.replace("_formed", "")
            os.environ["GDN_FORCE_VARIANT"] = base
            if plan.endswith("_formed"):
                os.environ["GDN_SEG_NO_TM"] = "1"
            else:
                os.environ.pop("GDN_SEG_NO_TM", None)
            if gdn.gdn_chunk_fwd_plan(B, T, Hk, Hv, dk, dv, C, gdn.GDN_BF16) != base:
                continue
            need = gdn.gdn_chunk_fwd_workspace_size(B, T, Hk, Hv, dk, dv, C, gdn.GDN_BF16)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
            call = lambda: gdn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"],
                                         initial_state=x["s0"], chunk=C, o=o, final_state=fs,
                                         workspace=ws)
            call()
            torch.cuda.synchronize()
            ts = []
            for _ in range(3):
                flush.fill_(1.0)
                e0, e1 = HipEvent(), HipEvent()
                e0.record(stream)
                call()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            ms = sorted(ts)[1]
            out[plan] = {"ms": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
                         "workspace_bytes": need}
            del ws
    finally:
        os.environ.pop("GDN_SEG_NO_TM", None)
        if old is None:
            os.environ.pop("GDN_FORCE_VARIANT", None)
        else:
            os.environ["GDN_FORCE_VARIANT"] = old
    del x, o, fs, flush
    torch.cuda.synchronize()
    return {"workload": c["name"], "plans": out,
            "default_plan": gdn.gdn_chunk_fwd_plan(B, T, Hk, Hv, dk, dv, C, gdn.GDN_BF16)}


# ------------------------------------------------------------------ peaks measured in the same run
def measured_peaks(torch, dev, stream):
    """What this GPU reaches on plain work, beside the vendor peaks: a 1 GiB device-to-device
    copy (read + write, GB/s) through torch and through the streaming-copy kernel of
    libgdn_calib.so (best of three grid sizes), a dense 8192^3 bf16 matrix product through
    torch/hipBLASLt, and the calibration library's loop of independent fp16 MFMAs (TFLOP/s).
    `copy_GBps` and `mfma_TFLOPs` are the best of each kind.  The copy kernel is tried with
    three grid sizes and four variants (grid-stride with 4 or 8 loads in flight, plain or
    non-temporal stores; one contiguous slice per workgroup),
    and as an in-place read + write of one 1 GiB buffer (the decode's access pattern)."""
    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        evs = [(HipEvent(), HipEvent()) for _ in range(reps)]
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return sorted(e0.elapsed_time(e1) for e0, e1 in evs)[reps // 2]
    n = 1 << 28
    src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    copy_ms = timed(lambda: dst.copy_(src))
    del src, dst
    m = 8192
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    a = torch.randn(m, m, device=dev, generator=g).to(torch.bfloat16)
    b = torch.randn(m, m, device=dev, generator=g).to(torch.bfloat16)
    mm_ms = timed(lambda: torch.matmul(a, b))
    del a, b
    torch.cuda.synchronize()
    import ctypes
    cal = ctypes.CDLL(os.path.join(ROOT, "linear_attention_token_gdn_amd", "libgdn_calib.so"))
    cal.gdn_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    cal.gdn_calib_mfma_clock.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    cal.gdn_calib_wall_clock_khz.restype = ctypes.c_int

    def ok(rc):
        if rc != 0:
            raise RuntimeError("calibration kernel failed (%d)" % rc)
    src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    hip_copy_ms = min(timed(lambda: ok(cal.gdn_calib_copy(src.data_ptr(), dst.data_ptr(), 4 * n,
                                                          blocks, var, stream.cuda_stream)))
                      for blocks in (1024, 2048, 4096) for var in (0, 1, 2, 4))
    upd_ms = min(timed(lambda: ok(cal.gdn_calib_copy(src.data_ptr(), src.data_ptr(), 4 * n,
                                                     blocks, 3, stream.cuda_stream)))
                 for blocks in (1024, 2048, 4096))
    del src, dst
    # the matrix-core loop in both product shapes (the same flops per round), with the engine
    # clock each workgroup's wavefront 0 saw: shader-clock cycles over wall-clock ticks
    blocks, iters = 2048, 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    clk = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
    wall_khz = cal.gdn_calib_wall_clock_khz()
    loop = {}
    for form in (0, 1):
        ms = timed(lambda: ok(cal.gdn_calib_mfma_clock(out.data_ptr(), clk.data_ptr(), blocks,
                                                        iters, form, stream.cuda_stream)))
        torch.cuda.synchronize()
        c = clk.view(blocks, 2).double().cpu()
        mhz = (c[:, 0] / c[:, 1]).median().item() * wall_khz / 1e3 if wall_khz > 0 else None
        loop[form] = (ms, mhz)
    del out, clk
    torch.cuda.synchronize()
    mfma_ms = loop[0][0]
    res = {"torch_copy_GBps": round(2 * n * 4 / (copy_ms * 1e-3) / 1e9, 1),
           "hip_copy_GBps": round(2 * n * 4 / (hip_copy_ms * 1e-3) / 1e9, 1),
           "hip_inplace_update_GBps": round(2 * n * 4 / (upd_ms * 1e-3) / 1e9, 1),
           "bf16_gemm_TFLOPs": round(2 * m ** 3 / (mm_ms * 1e-3) / 1e12, 1),
           "fp16_mfma_loop_TFLOPs": round(blocks * 4 * iters * 8 * 16384 / (mfma_ms * 1e-3) / 1e12, 1),
           "fp16_mfma32_loop_TFLOPs": round(blocks * 4 * iters * 4 * 32768 / (loop[1][0] * 1e-3) / 1e12, 1),
           "mfma_loop_sclk_MHz": [None if loop[f][1] is None else round(loop[f][1]) for f in (0, 1)],
           "what": "median of 5: 1 GiB device copy (torch; calibration kernel, best of 3 grids "
                   "x 4 variants); "
                   "8192 x 8192 x 8192 bf16 torch.matmul; 8 independent 16x16x32 fp16 MFMA "
                   "chains per wavefront (mfma32: 4 independent 32x32x16 chains), 8 wavefronts "
                   "per SIMD; mfma_loop_sclk_MHz: the engine clock during each loop (median "
                   "over workgroups of shader-clock cycles / wall-clock ticks)"}
    # the loop against the nominal peak scaled to the clock it ran at (the nominal dense fp16
    # peak assumes 2400 MHz)
    for f, key in ((0, "fp16_mfma_loop_TFLOPs"), (1, "fp16_mfma32_loop_TFLOPs")):
        if loop[f][1]:
            res.setdefault("mfma_loop_frac_of_nominal_at_clock", []).append(
                round(res[key] / (MFMA_BF16_PEAK_TFLOPS * loop[f][1] / 2400.0), 3))
    res["copy_GBps"] = max(res["torch_copy_GBps"], res["hip_copy_GBps"],
                           res["hip_inplace_update_GBps"])
    res["mfma_TFLOPs"] = max(res["bf16_gemm_TFLOPs"], res["fp16_mfma_loop_TFLOPs"],
                             res["fp16_mfma32_loop_TFLOPs"])
    return res


# ------------------------------------------------------------------ prologue / packed sequences
def _time(torch, stream, fn, reps=10):
    fn()
    torch.cuda.synchronize()
    evs = [(HipEvent(), HipEvent()) for _ in range(reps)]
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return sum(e0.elapsed_time(e1) for e0, e1 in evs) / reps


def prologue_and_packed(gdn, torch, dev, stream, pt, pc, o, fs):
    """(1) The prefill workload with the fused input prologue (q, k normalised and both gates
    taken as logits inside the kernels), against the same call on prepared inputs and against
    preparing them first with separate torch kernels.  (2) A packed batch: 32 sequences of
    seeded log-uniform lengths (64 .. 8192 tokens), 16 heads, d = 128, bf16, in one call."""
    import numpy as np
    allf = gdn.GDN_QK_L2NORM | gdn.GDN_BETA_LOGIT | gdn.GDN_G_LOGIT
    C = pc["chunk"]
    fused = lambda: gdn.chunk_fwd_varlen(pt["q"], pt["k"], pt["v"], pt["beta"], pt["g"],
                                         initial_state=pt["s0"], chunk=C, flags=allf, o=o,
                                         final_state=fs)
    F = torch.nn.functional

    def unfused():
        qn = F.normalize(pt["q"].float(), dim=-1).to(pt["q"].dtype)
        kn = F.normalize(pt["k"].float(), dim=-1).to(pt["k"].dtype)
        bt = torch.sigmoid(pt["beta"].float()).to(pt["beta"].dtype)
        gt = F.logsigmoid(pt["g"].float()).to(pt["g"].dtype)
        gdn.chunk_fwd(qn, kn, pt["v"], bt, gt, initial_state=pt["s0"], chunk=C, o=o,
                      final_state=fs)

    plain = lambda: gdn.chunk_fwd(pt["q"], pt["k"], pt["v"], pt["beta"], pt["g"],
                                  initial_state=pt["s0"], chunk=C, o=o, final_state=fs)
    plain_ms = _time(torch, stream, plain)  # standalone, like the two below
    fused_ms = _time(torch, stream, fused)
    unfused_ms = _time(torch, stream, unfused)
    B, T = pc["B"], pc["T"]
    res = {"prologue": {
        "workload": pc["name"], "flags": "qk_l2norm+beta_logit+g_logit",
        "fused_ms": round(fused_ms, 4), "plain_inputs_ms": round(plain_ms, 4),
        "separate_torch_prologue_ms": round(unfused_ms, 4),
        "fused_tokens_per_s": round(B * T / (fused_ms * 1e-3), 1)}}

    rng = np.random.Generator(np.random.PCG64(11))
    lengths = np.exp(rng.uniform(np.log(64), np.log(8192), 32)).astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    Tp, H, d = int(cu[-1]), 16, 128
    g = torch.Generator(device=dev)
    g.manual_seed(12)
    mk = lambda *shape: torch.randn(*shape, device=dev, generator=g).to(torch.bfloat16)
    q, k, v = mk(Tp, H, d), mk(Tp, H, d), mk(Tp, H, d)
    beta, ga = mk(Tp, H), mk(Tp, H) + 4.0
    cu_t = torch.from_numpy(cu).to(dev)
    ob = torch.empty((Tp, H, d), dtype=torch.float32, device=dev)
    sb = torch.empty((32, H, d, d), dtype=torch.float32, device=dev)
    packed = lambda: gdn.chunk_fwd_varlen(q, k, v, beta, ga, cu_seqlens=cu_t, chunk=64,
                                          flags=allf, o=ob, final_state=sb)
    packed_ms = _time(torch, stream, packed, reps=5)
    # the same batch with the plan hint for uneven lengths (split plan; workspace allocated once)
    hint = allf | gdn.GDN_PREFER_SPLIT
    hws = torch.empty(max(1, gdn.gdn_chunk_fwd_varlen_workspace_size(32, Tp, H, H, d, d, 64,
                                                                    gdn.GDN_BF16, 1, hint)),
                      dtype=torch.uint8, device=dev)
    packed_hint = lambda: gdn.chunk_fwd_varlen(q, k, v, beta, ga, cu_seqlens=cu_t, chunk=64,
                                               flags=hint, o=ob, final_state=sb, workspace=hws)
    packed_hint_ms = _time(torch, stream, packed_hint, reps=5)
    # backward of the prefill workload: all gradients, from a random gradient of o
    d_o = torch.randn(pt["v"].shape, device=dev, generator=g)
    bws = torch.empty(gdn.gdn_backward_workspace_size(B, T, pt["q"].shape[2], pt["v"].shape[2],
                                                      pt["q"].shape[3], pt["v"].shape[3]),
                      dtype=torch.uint8, device=dev)
    bwd = lambda: gdn.backward(pt["q"], pt["k"], pt["v"], pt["beta"], pt["g"], d_o,
                               initial_state=pt["s0"], workspace=bws)
    bwd_ms = _time(torch, stream, bwd, reps=3)
    res["backward"] = {"workload": pc["name"], "ms": round(bwd_ms, 3),
                       "tokens_per_s": round(B * T / (bwd_ms * 1e-3), 1),
                       "kernel": "bprep_kernel + bscan_kernel + bgrad_kernel (chunk-parallel MFMA; fp16 operands for bf16 inputs)"}
    res["packed"] = {"sequences": 32, "tokens": Tp, "min_len": int(lengths.min()),
                     "max_len": int(lengths.max()), "heads": H, "d": d, "dtype": "bf16",
                     "flags": "qk_l2norm+beta_logit+g_logit",
                     "ms": round(packed_ms, 4), "tokens_per_s": round(Tp / (packed_ms * 1e-3), 1),
                     "plan": "fused",
                     "with_split_hint": {"ms": round(packed_hint_ms, 4),
                                         "tokens_per_s": round(Tp / (packed_hint_ms * 1e-3), 1),
                                         "plan": "split (GDN_PREFER_SPLIT)"}}
    return res


EXP_PEAK_PER_S = 256 * 4 * 2.4e9 * 64 / 16  # v_exp_f32: a wave64 every 16 cycles per SIMD


def qsa_indexer(gdn, torch, dev, stream, with_cpu=True):
    """The QSA compressed indexer (gdn_qsa_index) on B=1, T=65536, 4 query heads and one key
    head of d=128 (bf16, seeded N(0,1)), r=4 (16384 blocks), 512 blocks (2048 tokens) kept,
    64 rotated dimensions.  The scoring and selection kernel is bound by the exponentials of
    the softmax, so its roofline is the vector units' exp rate.  The method needs one
    exponential per head and (query, block) pair, 4 per pair; the kernel evaluates them twice
    (once for the softmax normaliser, once for the importance) rather than storing them, and
    the roofline counts the 4 the method needs.  The fp64 oracle is timed on a sample of query
    rows."""
    B, T, d, r, nsel = 1, 65536, 128, 4, 512
    g = torch.Generator(device=dev)
    g.manual_seed(21)
    q = torch.randn(B, T, 4, d, device=dev, generator=g).to(torch.bfloat16)
    k = torch.randn(B, T, d, device=dev, generator=g).to(torch.bfloat16)
    ws = torch.empty(gdn.gdn_qsa_workspace_size(B, T, 4, d, r), dtype=torch.uint8, device=dev)
    sel = torch.empty(B, T, nsel, dtype=torch.int32, device=dev)
    call = lambda: gdn.qsa_index(q, k, r=r, nsel=nsel, rope_dims=64, sel=sel, workspace=ws)
    ms = _time(torch, stream, call, reps=5)
    nb = -(-T // r)
    pairs = sum(min((t + 1) // r, nb) for t in range(T - 1)) + nb  # eligible (query, block)
    res = {"workload": "B=1 T=65536 Hq=4 d=128 r=4 nsel=512 rope_dims=64 bf16",
           "ms": round(ms, 3), "queries_per_s": round(B * T / (ms * 1e-3), 1),
           "scored_pairs_per_s": round(pairs / (ms * 1e-3), 1),
           # one exponential per head and pair; the kernel performs each twice
           "roofline": {"bound": "alu", "unit": "exp/s", "peak": EXP_PEAK_PER_S,
                        "achieved": round(4 * pairs / (ms * 1e-3), 1),
                        "frac": round(4 * pairs / (ms * 1e-3) / EXP_PEAK_PER_S, 4),
                        "algorithmic_exps_per_pair": 4, "performed_exps_per_pair": 8,
                        "frac_performed": round(8 * pairs / (ms * 1e-3) / EXP_PEAK_PER_S, 4)},
           "score_TFLOPs_one_pass": round(2 * 4 * d * pairs / (ms * 1e-3) / 1e12, 2)}
    if with_cpu:
        import numpy as np
        from oracle import qsa as oq
        qn = q.float().cpu().numpy().astype(np.float64)
        kn = k.float().cpu().numpy().astype(np.float64)
        rows = np.linspace(T // 2, T - 1, 8).astype(np.int64)
        t0 = time.perf_counter()
        imp, elig = oq.importance(qn, kn, r, 64, 10000.0, 1.0 / d ** 0.5, rows=rows)
        oq.select(imp, elig, nsel)
        cpu_s = time.perf_counter() - t0
        pairs_s = sum(min((int(t) + 1) // r, nb) for t in rows)
        res["cpu_baseline"] = {"value": round(pairs_s / cpu_s, 1), "unit": "scored pairs/s",
                               "kind": "oracle", "cores": 1,  # numpy loops, one thread
                               "sample": "8 query rows in the second half of the sequence "
                                         "(keys pooled for the whole sequence)"}
    return res


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--prefill-config", type=int, default=3, choices=[1, 2, 3],
                    help="prefill workload: 3 = B1 T262144 H16 (default, the native context), "
                         "1 = B1 T4096 H16, 2 = B8 T8192 Hk16/Hv32")
    ap.add_argument("--cpu-sample-tokens", type=int, default=16384,
                    help="tokens of the prefill workload (all its chains) the oracle runs for "
                         "the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (known bytes, "
                         "to scale the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the input-prologue and packed-sequence measurements")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the Gated DeltaNet path here has no multi-GPU "
              "mode (--gpus %d requested); run with --gpus 1" % args.gpus, file=sys.stderr)
        return 2

    import torch
    import linear_attention_token_gdn_amd as gdn
    from gdn_inputs import CONFIGS, config_inputs

    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": nbytes, "calibrate_copy_bytes_written": nbytes,
                          "launches": 5}))
        return 0
    gdn.load_library()

    pc = CONFIGS[args.prefill_config]
    dc = CONFIGS[4]
    dec_inp = config_inputs(4)

    # ---- inputs resident in HBM
    pt = gpu_inputs(torch, dev, args.prefill_config)
    B, T, Hk, Hv, dk, dv, C = pc["B"], pc["T"], pc["Hk"], pc["Hv"], pc["dk"], pc["dv"], pc["chunk"]
    o = torch.empty((B, T, Hv, dv), dtype=torch.float32, device=dev)
    fs = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=dev)
    dt = dec_inp.to_torch(dev)
    nsteps_dec = dc["T"]
    dq = dt["q"].transpose(0, 1).contiguous()      # [64, B, H, d]: step s is a contiguous slice
    dk_ = dt["k"].transpose(0, 1).contiguous()
    dv_ = dt["v"].transpose(0, 1).contiguous()
    db = dt["beta"].transpose(0, 1).contiguous()
    dg = dt["g"].transpose(0, 1).contiguous()
    state = dt["s0"].clone()
    do = torch.empty((dc["B"], dc["Hv"], dc["dv"]), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def prefill():
        gdn.chunk_fwd(pt["q"], pt["k"], pt["v"], pt["beta"], pt["g"], initial_state=pt["s0"],
                      chunk=C, o=o, final_state=fs)

    def decode_all():
        for i in range(nsteps_dec):
            gdn.decode_step(dq[i], dk_[i], dv_[i], db[i], dg[i], state, o=do)

    for s in range(args.warmup):
        prefill()
        if not args.no_decode:
            decode_all()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = [[HipEvent() for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        e = ev[s]
        e[0].record(stream)
        prefill()
        e[1].record(stream)
        if not args.no_decode:
            e[2].record(stream)
            decode_all()
            e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    pre_ms = [e[0].elapsed_time(e[1]) for e in ev]
    pre_mean = sum(pre_ms) / len(pre_ms)
    pre_sorted = sorted(pre_ms)
    # the same call ten times back to back between one pair of events, with no decode traffic
    # around it (reported beside the in-step figure, which follows 64 decode launches)
    b2b = [HipEvent(), HipEvent()]
    b2b[0].record(stream)
    for _ in range(10):
        prefill()
    b2b[1].record(stream)
    torch.cuda.synchronize()
    b2b_ms = b2b[0].elapsed_time(b2b[1]) / 10
    flops = prefill_flops(B, T, Hk, Hv, dk, dv, C)
    pbytes = prefill_bytes(B, T, Hk, Hv, dk, dv, has_s0=pt["s0"] is not None)
    pre_tflops = flops / (pre_mean * 1e-3) / 1e12
    pre_gbs = pbytes / (pre_mean * 1e-3) / 1e9
    plan = gdn.gdn_chunk_fwd_plan(B, T, Hk, Hv, dk, dv, C, gdn.GDN_BF16)
    pre_kernels = {"split": "prep_kernel<%d,%d,false> + scan_kernel<%d,%d,float>" % (dk, C, dk, C),
                   "fused": "chunk_kernel<%d,%d,float,0>" % (dk, C),
                   # the transition pass storing each chunk's (I + A)^-1, the combine, the
                   # output pass reading it (modes 3 and 2; 1 and 0 with GDN_SEG_NO_TM)
                   "segmented": "chunk_kernel<%d,%d,float,%d> + seg_combine_kernel<%d> + "
                                "chunk_kernel<%d,%d,float,%d>" % (
                                    dk, C, 1 if os.environ.get("GDN_SEG_NO_TM") else 3, dk, dk, C,
                                    0 if os.environ.get("GDN_SEG_NO_TM") else 2)}.get(plan, plan)
    src_key = {"split": "prefill"}.get(plan, plan)
    rooflines = {
        "prefill": {
            "kernel": pre_kernels, "plan": plan, "bound": "hbm",
            "achieved": round(pre_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(pre_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(src_key, "workload%d" % args.prefill_config),
            "algorithmic_bytes": pbytes, "algorithmic_flops": flops,
            "mean_launch_ms": round(pre_mean, 4),
            "mfma_TFLOPs": round(pre_tflops, 2),
            "frac_bf16_mfma_peak": round(pre_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "mfma_counters": measured_mfma("workload%d_%s" % (args.prefill_config, plan),
                                           src_key),
        }
    }
    dom = "prefill"
    result_decode = None
    if not args.no_decode:
        dec_ms = [e[2].elapsed_time(e[3]) / nsteps_dec for e in ev]  # per decode launch
        dec_mean = sum(dec_ms) / len(dec_ms)
        sbytes, tbytes = decode_bytes(dc["B"], dc["Hk"], dc["Hv"], dc["dk"], dc["dv"])
        st_gbs = sbytes / (dec_mean * 1e-3) / 1e9
        tot_gbs = tbytes / (dec_mean * 1e-3) / 1e9
        rooflines["decode"] = {
            "kernel": "decode_kernel<%d,%d,bf16,float,false>" % (dc["dk"], dc["dv"]),
            "bound": "hbm",
            "achieved": round(tot_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(tot_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("decode", "workload4"),
            "algorithmic_bytes": tbytes, "mean_launch_ms": round(dec_mean, 4),
        }
        result_decode = {
            "state_GBps": round(st_gbs, 1), "frac_hbm_peak": round(st_gbs / HBM_PEAK_GBS, 4),
            "total_GBps": round(tot_gbs, 1),
            "us_per_step": round(dec_mean * 1e3, 2), "tokens_per_s": round(dc["B"] / (dec_mean * 1e-3), 1),
            "state_bytes_per_step": sbytes, "steps_per_bench_step": nsteps_dec,
        }
        if dec_mean * nsteps_dec > pre_mean:
            dom = "decode"

    # ---- several tokens per decode call (not part of the step): T tokens of the decode
    #      workload applied with one read and one write of every state (token by token for
    #      T < 5, as one chunk of the chunk form on the matrix cores from T = 5 on)
    multi = None
    if not args.no_decode:
        multi = {}
        st_out = torch.empty_like(state)
        for Tn, in_place in ((2, True), (4, True), (8, True), (8, False), (16, True)):
            mq, mk, mv = (dt[n][:, :Tn].contiguous() for n in ("q", "k", "v"))
            mb, mg = (dt[n][:, :Tn].contiguous() for n in ("beta", "g"))
            mo = torch.empty((dc["B"], Tn, dc["Hv"], dc["dv"]), dtype=torch.float32, device=dev)
            dst = state if in_place else st_out
            call = lambda: gdn.decode_tokens(mq, mk, mv, mb, mg, state, state_out=dst, o=mo)
            call()
            torch.cuda.synchronize()
            evs = [(HipEvent(), HipEvent()) for _ in range(5)]
            for e0, e1 in evs:
                e0.record(stream)
                call()
                e1.record(stream)
            torch.cuda.synchronize()
            ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / len(evs)
            sb, tb = decode_bytes(dc["B"], dc["Hk"], dc["Hv"], dc["dk"], dc["dv"], Tn)
            multi["T%d%s" % (Tn, "" if in_place else "_to_separate_state")] = {
                                 "kernel": "token" if Tn < 5 else "chunk (matrix cores)",
                                 "us_per_call": round(ms * 1e3, 2),
                                 "tokens_per_s": round(dc["B"] * Tn / (ms * 1e-3), 1),
                                 "state_GBps": round(sb / (ms * 1e-3) / 1e9, 1),
                                 "total_GBps": round(tb / (ms * 1e-3) / 1e9, 1),
                                 "frac_hbm_peak": round(tb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    # ---- the decode step over four state buffers in turn (not part of the step): each 512 MiB
    #      state is read again only after 1.5 GiB of other states, so the last-level cache
    #      (about 256 MB) cannot hold it between its reads
    cycled = None
    if not args.no_decode and not args.no_extras:
        states = [state] + [state.clone() for _ in range(3)]
        call = lambda: [gdn.decode_step(dq[i], dk_[i], dv_[i], db[i], dg[i], states[i % 4], o=do)
                        for i in range(nsteps_dec)]
        call()
        torch.cuda.synchronize()
        e0, e1 = HipEvent(), HipEvent()
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / nsteps_dec * 1e3
        sbytes, tbytes = decode_bytes(dc["B"], dc["Hk"], dc["Hv"], dc["dk"], dc["dv"])
        cycled = {"us_per_step": round(us, 2), "state_GBps": round(sbytes / (us * 1e-6) / 1e9, 1),
                  "total_GBps": round(tbytes / (us * 1e-6) / 1e9, 1),
                  "frac_hbm_peak": round(tbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                  "what": "64 decode steps, step i on state buffer i mod 4 (4 x 512 MiB)"}
        del states
        torch.cuda.synchronize()

    # ---- the input prologue, packed sequences and the backward, on the 4096-token workload
    #      (not part of the step)
    extras = None
    if not args.no_extras:
        xc = CONFIGS[1]
        xt = config_inputs(1).to_torch(dev)
        xo = torch.empty((xc["B"], xc["T"], xc["Hv"], xc["dv"]), dtype=torch.float32, device=dev)
        xfs = torch.empty((xc["B"], xc["Hv"], xc["dk"], xc["dv"]), dtype=torch.float32, device=dev)
        extras = prologue_and_packed(gdn, torch, dev, stream, xt, xc, xo, xfs)
        del xt, xo, xfs
    qsa = None if args.no_extras else qsa_indexer(gdn, torch, dev, stream,
                                                   with_cpu=not args.no_cpu_baseline)
    others = None if args.no_extras else prefill_configs(
        gdn, torch, dev, stream, names=[i for i in (1, 2, 3) if i != args.prefill_config])
    plans = None if args.no_extras else prefill_plans(gdn, torch, dev, stream, args.prefill_config)
    peaks = None if args.no_extras else measured_peaks(torch, dev, stream)
    if result_decode is not None and peaks is not None:
        result_decode["frac_measured_copy"] = round(result_decode["total_GBps"] / peaks["copy_GBps"], 4)
    # the binding roofline of the prefill: the larger of its HBM and MFMA times at peak
    t_bind = max(pbytes / (HBM_PEAK_GBS * 1e9), flops / (MFMA_BF16_PEAK_TFLOPS * 1e12))

    line = {
        "metric": "GDN prefill tokens/s + % bf16 MFMA peak; decode state GB/s % HBM peak",
        "value": round(B * T / (pre_mean * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 in, fp16 MFMA operands, fp32 accumulate/state",
        "data": "synthetic, seeded: the recipe's distributions (gdn_inputs recipe v1); prefill "
                "inputs drawn on the GPU with torch's generator, decode inputs by the recipe",
        "config": {
            "workload": pc["name"] + ("" if args.no_decode else " + " + dc["name"]),
            "prefill": {k_: pc[k_] for k_ in ("B", "T", "Hk", "Hv", "dk", "dv", "chunk", "dtype")},
            "decode": None if args.no_decode else
            {k_: dc[k_] for k_ in ("B", "Hk", "Hv", "dk", "dv", "dtype")},
        },
        "prefill": {"tokens_per_s": round(B * T / (pre_mean * 1e-3), 1),
                    "ms": round(pre_mean, 4), "TFLOPs": round(pre_tflops, 2),
                    "frac_bf16_mfma_peak": round(pre_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                    "GBps": round(pre_gbs, 1), "frac_hbm_peak": round(pre_gbs / HBM_PEAK_GBS, 4),
                    "back_to_back_ms": round(b2b_ms, 4),
                    "back_to_back_tokens_per_s": round(B * T / (b2b_ms * 1e-3), 1),
                    "ms_median": round(pre_sorted[len(pre_sorted) // 2], 4),
                    "ms_min": round(pre_sorted[0], 4),
                    "frac_binding_roofline": round(t_bind / (pre_mean * 1e-3), 4),
                    "frac_measured_gemm": None if peaks is None else
                    round(pre_tflops / peaks["bf16_gemm_TFLOPs"], 4),
                    "frac_measured_mfma": None if peaks is None else
                    round(pre_tflops / peaks["mfma_TFLOPs"], 4),
                    "frac_measured_copy": None if peaks is None else
                    round(pre_gbs / peaks["copy_GBps"], 4)},
        "decode": result_decode,
        "decode_cycled_states": cycled,
        "decode_tokens": multi,
        "prologue_and_packed": extras,
        "qsa_indexer": qsa,
        "prefill_other_workloads": others,
        "prefill_plans_compared": plans,
        "measured_peaks": peaks,
        "roofline": dict(rooflines[dom], kernel_role=dom),
        "rooflines": rooflines,
    }
    if not args.no_cpu_baseline:
        from gdn_inputs import make_inputs
        ts = min(T, args.cpu_sample_tokens)
        sample = make_inputs(B, ts, Hk, Hv, dk, dv, dtype=pc["dtype"], g_range=pc["g_range"],
                             s0_std=pc["s0_std"], seed=pc["seed"])
        line["cpu_baseline"] = cpu_baseline(sample, dec_inp, T)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
