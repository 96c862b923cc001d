"""Seeded synthetic inputs for the gated delta rule workloads.

This module is the only code shared by the GPU library's tests/benchmark and
the fp64 oracle: it draws random inputs and holds none of the method's
arithmetic.  Values are returned as float32 numpy arrays that hold exactly the
stored values (for bf16 workloads, bf16 values widened to float32), so both
sides consume bit-identical inputs.

Recipe (a repository convention; the pages give no activation statistics):
  * numpy Generator(PCG64(seed)); draws in float32.
  * if the workload has an initial state: S0 ~ N(0, std^2) drawn first, shape
    [B, Hv, dk, dv], kept in float32 (the state is always float32).
  * then, per block of up to 8192 tokens (t0 = 0, 8192, ...), in this order:
    q [B, blk, Hk, dk], k (same), v [B, blk, Hv, dv], beta-logit [B, blk, Hv],
    u [B, blk, Hv] ~ U(lo, hi).
  * q and k are divided by their L2 norm over the head dimension in float64
    (no epsilon), then rounded to the storage dtype.
  * beta = sigmoid(beta-logit) computed in float64, then rounded.
  * g = log(alpha) = -u, rounded to the storage dtype.
  * rounding to bf16 is round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BLOCK_T = 8192
RECIPE_VERSION = 1


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even); result is float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    r = (b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x)
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "bf16":
        return round_to_bf16(x.astype(np.float32))
    raise ValueError("unknown dtype %r" % dtype)


@dataclasses.dataclass
class GdnInputs:
    """Stored input values of one workload (float32 arrays holding exact stored values)."""
    q: np.ndarray          # [B, T, Hk, dk]
    k: np.ndarray          # [B, T, Hk, dk]
    v: np.ndarray          # [B, T, Hv, dv]
    beta: np.ndarray       # [B, T, Hv]
    g: np.ndarray          # [B, T, Hv]   (log alpha, <= 0)
    s0: Optional[np.ndarray]  # [B, Hv, dk, dv] float32 or None
    dtype: str             # storage dtype of q, k, v, beta, g: "f32" or "bf16"

    @property
    def shape(self):
        B, T, Hk, dk = self.q.shape
        return dict(B=B, T=T, Hk=Hk, Hv=self.v.shape[2], dk=dk, dv=self.v.shape[3])

    def to_torch(self, device, with_state=True):
        """Torch tensors in the storage dtype on ``device`` (exact conversion)."""
        import torch
        dt = torch.bfloat16 if self.dtype == "bf16" else torch.float32

        def cv(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(device=device).to(dt)

        out = dict(q=cv(self.q), k=cv(self.k), v=cv(self.v), beta=cv(self.beta), g=cv(self.g))
        if with_state:
            out["s0"] = (None if self.s0 is None else
                         torch.from_numpy(np.ascontiguousarray(self.s0)).to(device=device))
        return out


def make_inputs(B, T, Hk, Hv, dk, dv, dtype="bf16", g_range=(0.001, 0.2),
                s0_std=None, seed=0) -> GdnInputs:
    """Draw one workload's inputs following the recipe in the module docstring."""
    rng = np.random.Generator(np.random.PCG64(seed))
    s0 = None
    if s0_std is not None:
        s0 = (rng.standard_normal((B, Hv, dk, dv), dtype=np.float32) * np.float32(s0_std)).astype(np.float32)
    q = np.empty((B, T, Hk, dk), np.float32)
    k = np.empty((B, T, Hk, dk), np.float32)
    v = np.empty((B, T, Hv, dv), np.float32)
    beta = np.empty((B, T, Hv), np.float32)
    g = np.empty((B, T, Hv), np.float32)
    lo, hi = g_range
    for t0 in range(0, T, BLOCK_T):
        n = min(BLOCK_T, T - t0)
        for dst, d, H in ((q, dk, Hk), (k, dk, Hk)):
            x = rng.standard_normal((B, n, H, d), dtype=np.float32).astype(np.float64)
            x /= np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
            dst[:, t0:t0 + n] = round_to(x, dtype)
        v[:, t0:t0 + n] = round_to(rng.standard_normal((B, n, Hv, dv), dtype=np.float32), dtype)
        logit = rng.standard_normal((B, n, Hv), dtype=np.float32).astype(np.float64)
        beta[:, t0:t0 + n] = round_to(1.0 / (1.0 + np.exp(-logit)), dtype)
        u = rng.uniform(lo, hi, size=(B, n, Hv)).astype(np.float32)
        g[:, t0:t0 + n] = round_to(-u, dtype)
    return GdnInputs(q=q, k=k, v=v, beta=beta, g=g, s0=s0, dtype=dtype)


# The five workloads.  "steps" marks the decode workload: its inputs are drawn
# as a T = steps sequence and decode step s consumes token s.
CONFIGS = {
    0: dict(name="tiny_f32_b1_t64_h2_d16_c16", kind="prefill", B=1, T=64, Hk=2, Hv=2,
            dk=16, dv=16, chunk=16, dtype="f32", g_range=(0.001, 0.2), s0_std=None, seed=0),
    1: dict(name="prefill_bf16_b1_t4096_h16_d128_c64", kind="prefill", B=1, T=4096, Hk=16,
            Hv=16, dk=128, dv=128, chunk=64, dtype="bf16", g_range=(0.001, 0.2),
            s0_std=None, seed=1),
    2: dict(name="prefill_gqa_bf16_b8_t8192_hk16_hv32_d128_c64", kind="prefill", B=8, T=8192,
            Hk=16, Hv=32, dk=128, dv=128, chunk=64, dtype="bf16", g_range=(0.001, 0.2),
            s0_std=0.02, seed=2),
    3: dict(name="prefill_long_bf16_b1_t262144_h16_d128_c64", kind="prefill", B=1, T=262144,
            Hk=16, Hv=16, dk=128, dv=128, chunk=64, dtype="bf16", g_range=(0.0001, 0.02),
            s0_std=None, seed=3),
    4: dict(name="decode_bf16_b256_h32_d128_64steps", kind="decode", B=256, T=64, Hk=32,
            Hv=32, dk=128, dv=128, chunk=None, dtype="bf16", g_range=(0.001, 0.2),
            s0_std=0.02, seed=4),
}


def config_inputs(idx: int) -> GdnInputs:
    c = CONFIGS[idx]
    return make_inputs(c["B"], c["T"], c["Hk"], c["Hv"], c["dk"], c["dv"], dtype=c["dtype"],
                       g_range=c["g_range"], s0_std=c["s0_std"], seed=c["seed"])
