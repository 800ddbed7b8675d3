"""Seeded synthetic inputs for the flash-attention training forward.

This module is shared by the oracle side (tests, CPU baseline) and the GPU
side (tests, bench, smoke) and holds none of the attention arithmetic: it
turns (workload, seed) into bf16 Q/K/V bit patterns and an optional f32
additive mask, through the counter-based generator in fagen.c.

Workloads (every tensor contiguous, row-major):
  Q [B,H,ql,D], K/V [B,Hkv,kl,D] as bf16 bits (numpy uint16);
  mask [B,H,ql,kl] f32 (0 or -inf) or None.
"""
import ctypes
import math
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

# The seed constant of the method's test page ("TRAIN001" in ASCII), used as
# the base seed; each workload adds its own offset.
SEED_BASE = 0x5452_4149_4E30_3031

STREAM_Q, STREAM_K, STREAM_V, STREAM_MASK, STREAM_ROWS = 0, 1, 2, 3, 4

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.fagen_normal_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double,
                                          ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int]
        lib.fagen_normal_bf16.restype = ctypes.c_int
        lib.fagen_mask_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                       ctypes.c_double, ctypes.c_int, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_void_p]
        lib.fagen_mask_f32.restype = ctypes.c_int
        lib.fagen_word.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64]
        lib.fagen_word.restype = ctypes.c_uint64
        lib.fagen_lcg_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p]
        lib.fagen_lcg_f32.restype = None
        lib.fagen_lcg_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p]
        lib.fagen_lcg_bf16.restype = None
        _lib = lib
    return _lib


def default_threads():
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def word(seed, stream, i):
    """The raw 64-bit word number i of a stream (for tests of the generator)."""
    return int(_load().fagen_word(seed & (2**64 - 1), stream, i))


def normal_bf16(seed, stream, shape, sigma=1.0, n_threads=None):
    """iid N(0, sigma^2) values rounded to bf16; returns uint16 bits of `shape`."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16)
    rc = _load().fagen_normal_bf16(seed & (2**64 - 1), stream, float(sigma),
                                   out.ctypes.data if n else None, n,
                                   n_threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"fagen_normal_bf16 failed ({rc})")
    return out.reshape(shape)


def mask_f32(seed, B, H, ql, kl, p_masked=0.1, n_full_rows=4):
    """Additive f32 mask [B,H,ql,kl]: -inf w.p. p_masked else 0, plus n_full_rows
    distinct fully -inf rows per (b,h). Returns (mask, full_rows[B,H,n_full_rows])."""
    mask = np.empty((B, H, ql, kl), dtype=np.float32)
    rows = np.empty((B, H, n_full_rows), dtype=np.int32)
    rc = _load().fagen_mask_f32(seed & (2**64 - 1), STREAM_MASK, STREAM_ROWS, float(p_masked),
                                int(n_full_rows), B, H, ql, kl,
                                mask.ctypes.data if mask.size else None,
                                rows.ctypes.data if rows.size else None)
    if rc != 0:
        raise RuntimeError(f"fagen_mask_f32 failed ({rc})")
    return mask, rows


def lcg_f32(seed, shape):
    """The method's test inputs: values of its test page's 64-bit LCG from
    `seed` (pseudo_random_f32 there), f32 in [-0.5, 0), of `shape`."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32)
    if n:
        _load().fagen_lcg_f32(seed & (2**64 - 1), n, out.ctypes.data)
    return out.reshape(shape)


def lcg_bf16(seed, shape):
    """lcg_f32 rounded to bf16 (round to nearest even); uint16 bits of `shape`."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16)
    if n:
        _load().fagen_lcg_bf16(seed & (2**64 - 1), n, out.ctypes.data)
    return out.reshape(shape)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Hkv: int
    ql: int
    kl: int
    D: int
    causal: bool
    sigma: float = 1.0
    mask_p: float = None        # None: no additive mask
    mask_full_rows: int = 0
    seed_offset: int = 0

    @property
    def seed(self):
        return (SEED_BASE + self.seed_offset) & (2**64 - 1)

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.D)

    @property
    def metric_flop(self):
        """4*B*H*ql*kl*D, halved for causal (the reported-throughput convention)."""
        f = 4 * self.B * self.H * self.ql * self.kl * self.D
        return f // 2 if self.causal else f

    def with_(self, **kw):
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five workloads of the forward pass, from the smallest (the oracle runs it
# whole in well under a second) to the training- and long-context-scale ones.
WORKLOADS = {
    w.name: w for w in [
        Workload("d64_b1_h2_q64_k64", 1, 2, 2, 64, 64, 64, False, seed_offset=0),
        Workload("d256_gqa_b2_h8kv2_q128_k128_causal", 2, 8, 2, 128, 128, 256, True, seed_offset=1),
        Workload("d64_mask_b2_h4_q64_k256_causal", 2, 4, 4, 64, 256, 64, True,
                 mask_p=0.1, mask_full_rows=4, seed_offset=2),
        Workload("d64_b8_h16_q4096_k4096_causal", 8, 16, 16, 4096, 4096, 64, True, seed_offset=3),
        Workload("d256_gqa_b2_h16kv4_q8192_k8192_causal", 2, 16, 4, 8192, 8192, 256, True,
                 sigma=0.5, seed_offset=4),
    ]
}
WORKLOAD_ORDER = list(WORKLOADS)


def generate(w, n_threads=None):
    """Inputs of workload `w`: dict with q, k, v (uint16 bf16 bits), mask (f32 or
    None) and full_rows (int32 [B,H,n] or None)."""
    q = normal_bf16(w.seed, STREAM_Q, (w.B, w.H, w.ql, w.D), w.sigma, n_threads)
    k = normal_bf16(w.seed, STREAM_K, (w.B, w.Hkv, w.kl, w.D), w.sigma, n_threads)
    v = normal_bf16(w.seed, STREAM_V, (w.B, w.Hkv, w.kl, w.D), w.sigma, n_threads)
    mask = rows = None
    if w.mask_p is not None:
        mask, rows = mask_f32(w.seed, w.B, w.H, w.ql, w.kl, w.mask_p, w.mask_full_rows)
    return dict(q=q, k=k, v=v, mask=mask, full_rows=rows)


def bf16_bits_to_f32(bits):
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
