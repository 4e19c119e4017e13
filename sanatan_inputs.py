"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and the CPU oracle.

This module holds no arithmetic of the attention method: it draws q, k, v ~ N(0,1), the
per-head root anchors omega ~ U(-pi, pi), and rounds to bfloat16 where a workload is bf16.
Both sides consume exactly these values (the oracle upcasts them to fp64).

Recipe (numpy PCG64 ``default_rng(seed)``; float64 draws -> float32 -> RNE to bf16 where
the workload says bf16):  draw order q, k, v, then omega.  Decode workloads draw omega first,
then the state-filling tokens (q, k, v), then the decode tokens (q, k, v per step).
Very large decode batches are drawn on the GPU with torch's seeded Philox generator instead
(numpy would need minutes); the oracle then receives copies of the sampled heads' inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D_HEAD = 64


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(shape).astype(np.float32)
    return bf16_round(x) if dtype == "bf16" else x


def _omega(rng: np.random.Generator, rows: int, d: int) -> np.ndarray:
    return rng.uniform(-np.pi, np.pi, size=(rows, d)).astype(np.float32)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    H: int
    T: int
    dtype: str                  # "f32" or "bf16"
    chunk: int = 64
    p: int = 1
    d: int = D_HEAD
    dv: int = D_HEAD
    gamma: float = 4.0
    lambda_base: float = 10000.0
    eps: float = 1e-6
    extra: dict = field(default_factory=dict)


# The five named workloads (shapes, dtypes, chunk sizes and seeds).
TINY = Workload("tiny_b1h1_t256_f32", 1000, 1, 1, 256, "f32", chunk=64)
PREFILL = Workload("prefill_b8h12_t2048_bf16", 1001, 8, 12, 2048, "bf16", chunk=64)
DECODE = Workload("decode_l12h12_fill4096_steps1024_f32", 1002, 1, 144, 4096, "f32",
                  extra={"steps": 1024, "batches": (1, 64)})
LONG = Workload("long_prefill_b1h12_t32768_bf16", 1003, 1, 12, 32768, "bf16", chunk=128)
QUAD_P2 = Workload("quadratic_p2_b4h12_t4096_bf16", 1004, 4, 12, 4096, "bf16", p=2)
WORKLOADS = {w.name: w for w in (TINY, PREFILL, DECODE, LONG, QUAD_P2)}


def attention_inputs(seed: int, B: int, H: int, T: int, dtype: str, d: int = D_HEAD, dv: int = D_HEAD):
    """q, k [B,H,T,d], v [B,H,T,dv] (float32 arrays, bf16-exact when dtype == 'bf16'), omega [H,d]."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (B, H, T, d), dtype)
    k = _normal(rng, (B, H, T, d), dtype)
    v = _normal(rng, (B, H, T, dv), dtype)
    omega = _omega(rng, H, d)
    return q, k, v, omega


def workload_inputs(w: Workload):
    return attention_inputs(w.seed, w.B, w.H, w.T, w.dtype, w.d, w.dv)


def decode_inputs_numpy(seed: int, n_heads: int, fill: int, steps: int, d: int = D_HEAD, dv: int = D_HEAD):
    """Batch-1 decode inputs: omega [n_heads,d]; fill tokens q,k [n_heads,fill,d], v [..,dv];
    decode tokens q,k [steps,n_heads,d], v [steps,n_heads,dv] (float32)."""
    rng = np.random.default_rng(seed)
    omega = _omega(rng, n_heads, d)
    fq = _normal(rng, (n_heads, fill, d), "f32")
    fk = _normal(rng, (n_heads, fill, d), "f32")
    fv = _normal(rng, (n_heads, fill, dv), "f32")
    sq = _normal(rng, (steps, n_heads, d), "f32")
    sk = _normal(rng, (steps, n_heads, d), "f32")
    sv = _normal(rng, (steps, n_heads, dv), "f32")
    return omega, (fq, fk, fv), (sq, sk, sv)


def decode_positions(seed: int, n: int, lo: int = 0, hi: int = 1 << 20) -> np.ndarray:
    """Per head-state positions for a batch of sequences at different lengths: int64 [n], uniform in [lo, hi)."""
    return np.random.default_rng(seed).integers(lo, hi, size=n, dtype=np.int64)


def decode_inputs_torch(seed: int, batch: int, n_heads: int, fill: int, steps: int, device, d: int = D_HEAD,
                        dv: int = D_HEAD):
    """Large-batch decode inputs drawn on `device` with torch's seeded generator.

    omega [n_heads,d] comes from numpy (same recipe as above); fill tokens are
    [batch*n_heads, fill, d]; decode tokens [steps, batch*n_heads, d].  float32.
    """
    import torch

    rng = np.random.default_rng(seed)
    omega = _omega(rng, n_heads, d)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    N = batch * n_heads
    kw = dict(generator=g, device=device, dtype=torch.float32)
    fq = torch.randn((N, fill, d), **kw)
    fk = torch.randn((N, fill, d), **kw)
    fv = torch.randn((N, fill, dv), **kw)
    sq = torch.randn((steps, N, d), **kw)
    sk = torch.randn((steps, N, d), **kw)
    sv = torch.randn((steps, N, dv), **kw)
    return omega, (fq, fk, fv), (sq, sk, sv)
