"""Seeded synthetic inputs for the fixed-m attention workloads.

This module only draws and lays out input tensors.  It holds none of the attention
method's arithmetic (no norms-for-bounds, no shift, no gate, no softmax), so both the HIP
path's tests and the fp64 oracle can take their inputs from it.

The shapes follow the Wan2.2 self-attention that the pages measure on: 40 heads of
head_dim 128, and for the 720p one-rank share 18,900 resident query tokens against
75,600 keys visited as 4 ring chunks ([CM] Overview; [FM] fallback-rate table, N = 75,600).
The Wan2.2 weights and the VBench prompts are not available; these seeded tensors stand in
for the activations at the real shapes.  Per-row RMS normalisation mimics the model's
QK-norm, which is what keeps per-token norm spread bounded ([CM] "Adapting this kernel").

Recipe: numpy PCG64 with SeedSequence(1000 + config id).spawn(4) for (q, k, v, mu);
standard normals drawn in fp32; RMS normalisation x / sqrt(mean(x^2)) in fp32; then
round-to-nearest-even to bf16 for the bf16 workloads.  Layout [B, S, H, D].

  [CM] "Kernel reference: ring_attention_const_max_fwd const-max ring attention"
  [FM] "feat(attention): fixed-m splash attention kernel with dynamic bounds and safety
       fallbacks" (maxdiffusion pull request #477)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "bf16_bits_from_f32", "f32_from_bf16_bits",
           "Inputs", "make_inputs", "generic_inputs"]


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    dtype: str                  # "bf16" or "fp32"
    batch: int
    heads: int
    head_dim: int
    sq: int
    chunks: tuple               # K/V chunk lengths in visit order
    q_block: int
    center: str                 # "none" | "supplied" | "compute"
    recipe: str

    @property
    def sk(self) -> int:
        return int(sum(self.chunks))

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def flops(self) -> float:
        """4 * B * H * Sq * Sk * D: the two matmuls of attention, 2 flop per MAC."""
        return 4.0 * self.batch * self.heads * self.sq * self.sk * self.head_dim


WORKLOADS = {
    1: Workload(1, "tiny-fp32", "fp32", 1, 1, 64, 256, (128, 128), 256, "none",
                "q,k,v iid N(0,1); scale 1/8; 2 chunks of 128"),
    2: Workload(2, "wan-block-bf16", "bf16", 1, 40, 128, 4096, (1024,) * 4, 256, "none",
                "q,k rows RMS-normalised (norm sqrt(128)), v N(0,1); scale 1/sqrt(128)"),
    3: Workload(3, "wan720p-rank-share-bf16", "bf16", 1, 40, 128, 18900, (18900,) * 4, 256,
                "compute", "q,k,v rows RMS-normalised per head; global k_mean computed"),
    4: Workload(4, "ragged-offset-bf16", "bf16", 1, 40, 128, 4096, (37800,), 256, "supplied",
                "q,v N(0,1); k = mu_h + N(0,1) with |mu_h| = 3; k_mean supplied = mu"),
    5: Workload(5, "adversarial-gate-fp32", "fp32", 1, 8, 128, 4096, (1024,) * 4, 256, "none",
                "heads 0-3 iid N(0,1); heads 4-7: keys exactly centred with max centred "
                "norm 1, queries of base-2 norm 231.01"),
}


def get(cid: int) -> Workload:
    return WORKLOADS[cid]


# --------------------------------------------------------------------------------------
# bf16 storage helpers (numpy has no bf16: bf16 tensors are carried as uint16 bit patterns)
# --------------------------------------------------------------------------------------
def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even), returned as uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Inputs:
    """One workload's tensors.  For bf16, *_store hold uint16 bit patterns and the f32
    views are their exact widening; for fp32 both are the same float32 arrays."""
    wl: Workload
    q_store: np.ndarray
    k_store: list
    v_store: list
    k_mean: np.ndarray | None = None          # supplied fp32 [B, H, D] (center == supplied)
    extra: dict = field(default_factory=dict)

    def _f32(self, a):
        return f32_from_bf16_bits(a) if self.wl.dtype == "bf16" else a

    @property
    def q(self) -> np.ndarray:
        return self._f32(self.q_store)

    @property
    def k(self) -> list:
        return [self._f32(c) for c in self.k_store]

    @property
    def v(self) -> list:
        return [self._f32(c) for c in self.v_store]


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _rms_rows(x):
    """x / sqrt(mean(x^2)) over the last axis, in fp32."""
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=np.float32)
    return (x / np.sqrt(ms)).astype(np.float32)


def _store(x, dtype):
    return bf16_bits_from_f32(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def _split(x, lens):
    out, lo = [], 0
    for n in lens:
        out.append(np.ascontiguousarray(x[:, lo:lo + n]))
        lo += n
    return out


def make_inputs(cid: int) -> Inputs:
    """Draw the inputs of workload `cid` (identical bytes on every call and machine)."""
    wl = WORKLOADS[cid]
    sq_seed, sk_seed, sv_seed, smu_seed = np.random.SeedSequence(1000 + cid).spawn(4)
    rq, rk, rv, rmu = (np.random.Generator(np.random.PCG64(s))
                       for s in (sq_seed, sk_seed, sv_seed, smu_seed))
    B, H, D, Sq, N = wl.batch, wl.heads, wl.head_dim, wl.sq, wl.sk
    k_mean = None
    extra = {}
    if cid == 1:
        q, k, v = _normal(rq, (B, Sq, H, D)), _normal(rk, (B, N, H, D)), _normal(rv, (B, N, H, D))
    elif cid == 2:
        q = _rms_rows(_normal(rq, (B, Sq, H, D)))
        k = _rms_rows(_normal(rk, (B, N, H, D)))
        v = _normal(rv, (B, N, H, D))
    elif cid == 3:
        q = _rms_rows(_normal(rq, (B, Sq, H, D)))
        k = _rms_rows(_normal(rk, (B, N, H, D)))
        v = _rms_rows(_normal(rv, (B, N, H, D)))
    elif cid == 4:
        mu = _normal(rmu, (B, H, D))
        mu = (mu * (np.float32(3.0) / np.linalg.norm(mu, axis=-1, keepdims=True))).astype(np.float32)
        q = _normal(rq, (B, Sq, H, D))
        k = (_normal(rk, (B, N, H, D)) + mu[:, None, :, :]).astype(np.float32)
        v = _normal(rv, (B, N, H, D))
        k_mean = mu.astype(np.float32)
    elif cid == 5:
        q = _normal(rq, (B, Sq, H, D))
        k = _normal(rk, (B, N, H, D))
        v = _normal(rv, (B, N, H, D))
        # Heads 4-7: keys centred exactly (fp64 mean removed) and scaled so the largest
        # centred key norm is 1; every query row gets norm 231.01 in base-2 exponent
        # units, i.e. |q| = 231.01 / (scale * log2 e).  [FM] "Why the gate is halved".
        k64 = k[:, :, 4:].astype(np.float64)
        k64 = k64 - k64.mean(axis=1, keepdims=True)
        k64 = k64 / np.linalg.norm(k64, axis=-1).max(axis=1)[:, None, :, None]
        k[:, :, 4:] = k64.astype(np.float32)
        qnorm = 231.01 / (float(np.float32(wl.scale)) * 1.4426950408889634)
        q64 = q[:, :, 4:].astype(np.float64)
        q64 = q64 / np.linalg.norm(q64, axis=-1, keepdims=True) * qnorm
        q[:, :, 4:] = q64.astype(np.float32)
        extra["adversarial_heads"] = (4, 5, 6, 7)
        extra["query_base2_norm"] = 231.01
    else:
        raise KeyError(cid)
    return Inputs(wl, _store(q, wl.dtype), _split(_store(k, wl.dtype), wl.chunks),
                  _split(_store(v, wl.dtype), wl.chunks), k_mean, extra)


def generic_inputs(seed: int, dtype: str, B: int, H: int, D: int, Sq: int, chunks,
                   q_block: int = 64, center: str = "none", q_scale: float = 1.0,
                   k_offset: float = 0.0) -> Inputs:
    """Small seeded inputs of any shape for edge-case tests: q, k, v iid N(0,1) with q
    multiplied by q_scale and, if k_offset > 0, a shared per-head key offset of that norm."""
    wl = Workload(0, f"generic-{seed}", dtype, B, H, D, Sq, tuple(int(c) for c in chunks),
                  q_block, center, "generic")
    rq, rk, rv, rmu = (np.random.Generator(np.random.PCG64(s))
                       for s in np.random.SeedSequence(seed).spawn(4))
    N = wl.sk
    q = (_normal(rq, (B, Sq, H, D)) * np.float32(q_scale)).astype(np.float32)
    k = _normal(rk, (B, N, H, D))
    v = _normal(rv, (B, N, H, D))
    k_mean = None
    if k_offset > 0:
        mu = _normal(rmu, (B, H, D))
        mu = (mu * (np.float32(k_offset) / np.linalg.norm(mu, axis=-1, keepdims=True))).astype(np.float32)
        k = (k + mu[:, None]).astype(np.float32)
        k_mean = mu
    return Inputs(wl, _store(q, dtype), _split(_store(k, dtype), wl.chunks),
                  _split(_store(v, dtype), wl.chunks), k_mean)
