"""Plain CPU reference (oracle) for the flash-attention training forward
and its backward.

TEST INFRASTRUCTURE ONLY: only tests/, the smoke check of __graft_entry__ and
the bench's cpu_baseline leg may import this package. It shares no code with
the GPU path (flash_attention_forward_fa_amd) and never imports it.

The arithmetic lives in fa_oracle.c: softmax attention and its logsumexp
written from their definition in single precision (the operation of the
method's page, "mlx-native 0.9.0", tests/test_flash_attn_train.rs, section
"CPU oracle - forward O + logsumexp L"), and the FA-2 backward of the same
page's "Phase 2 - backward kernel helpers". This wrapper widens bf16 inputs
to f32 (exact), calls it, and rounds O to bf16 the way that page's
oracle_for_bf16 helper does.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _bind(path):
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.fa_oracle_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                  ctypes.c_float, ctypes.c_int, vp, vp, ctypes.c_int]
    lib.fa_oracle_fwd.restype = ctypes.c_int
    lib.fa_oracle_fwd_rows.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                       ctypes.c_float, ctypes.c_int, vp, i64, vp, vp,
                                       ctypes.c_int]
    lib.fa_oracle_fwd_rows.restype = ctypes.c_int
    lib.fa_oracle_fwd_swa.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                      ctypes.c_float, i64, vp, i64, vp, vp, ctypes.c_int]
    lib.fa_oracle_fwd_swa.restype = ctypes.c_int
    lib.fa_oracle_fwd_general.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                          ctypes.c_float, ctypes.c_int, i64, vp, i64, vp, vp,
                                          ctypes.c_int]
    lib.fa_oracle_fwd_general.restype = ctypes.c_int
    lib.fa_oracle_fwd_sinks.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                        ctypes.c_float, ctypes.c_int, i64, vp, vp, i64, vp, vp,
                                        ctypes.c_int]
    lib.fa_oracle_fwd_sinks.restype = ctypes.c_int
    lib.fa_oracle_bwd_general.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                          i64, ctypes.c_float, ctypes.c_int, i64, vp, i64, vp, vp,
                                          vp, ctypes.c_int]
    lib.fa_oracle_bwd_general.restype = ctypes.c_int
    lib.fa_oracle_round_bf16.argtypes = [vp, vp, i64]
    lib.fa_oracle_round_bf16.restype = None
    lib.fa_oracle_bwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                  ctypes.c_float, ctypes.c_int, vp, vp, vp, ctypes.c_int]
    lib.fa_oracle_bwd.restype = ctypes.c_int
    lib.fa_oracle_bwd_swa.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                      ctypes.c_float, ctypes.c_int, i64, vp, vp, vp, ctypes.c_int]
    lib.fa_oracle_bwd_swa.restype = ctypes.c_int
    lib.fa_oracle_bwd_sinks.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                        i64, ctypes.c_float, ctypes.c_int, i64, vp, vp,
                                        ctypes.c_int]
    lib.fa_oracle_bwd_sinks.restype = ctypes.c_int
    lib.fa_oracle_bwd_given_o.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                          i64, i64, ctypes.c_float, ctypes.c_int, i64, vp, vp,
                                          vp, ctypes.c_int]
    lib.fa_oracle_bwd_given_o.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = _bind(_build.LIB)
    return _lib


def default_threads():
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def widen_bf16(bits):
    """bf16 bit patterns (uint16) -> float32 values, exact."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_bf16(x, lib=None):
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    if x.size:
        (lib or _load()).fa_oracle_round_bf16(x.ctypes.data, out.ctypes.data, x.size)
    return out


def _f32(a):
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return widen_bf16(a)
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None or a.size == 0 else a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what} rejected its arguments (code {rc})")


def fwd(q, k, v, mask, B, H, Hkv, ql, kl, D, scale, causal, n_threads=None, lib=None,
        window=None):
    """Full forward. q/k/v: bf16 bits (uint16) or float32 arrays; mask f32 or None.
    window: None, or a sliding window (>= 0, implies the causal rule).

    Returns (O_f32 [B,H,ql,D], O_bf16_bits [B,H,ql,D], L [B,H,ql])."""
    qf, kf, vf, mf = _f32(q), _f32(k), _f32(v), _f32(mask)
    O = np.empty((B, H, ql, D), dtype=np.float32)
    L = np.empty((B, H, ql), dtype=np.float32)
    lib = lib or _load()
    if window is not None:
        rc = lib.fa_oracle_fwd_swa(_ptr(qf), _ptr(kf), _ptr(vf), _ptr(mf), B, H, Hkv, ql, kl,
                                   D, float(scale), int(window), None, 0, _ptr(O), _ptr(L),
                                   n_threads or default_threads())
        _check(rc, "fa_oracle_fwd_swa")
        return O, round_bf16(O, lib), L
    rc = lib.fa_oracle_fwd(_ptr(qf), _ptr(kf), _ptr(vf), _ptr(mf), B, H, Hkv, ql, kl, D,
                               float(scale), int(bool(causal)), _ptr(O), _ptr(L),
                               n_threads or default_threads())
    _check(rc, "fa_oracle_fwd")
    return O, round_bf16(O, lib), L


def fwd_rows(q, k, v, mask, B, H, Hkv, ql, kl, D, scale, causal, rows, n_threads=None,
             lib=None, window=None):
    """Selected flat rows ((b*H + h)*ql + i). Returns (O_f32 [n,D], O_bf16 [n,D], L [n])."""
    qf, kf, vf, mf = _f32(q), _f32(k), _f32(v), _f32(mask)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = rows.size
    O = np.empty((n, D), dtype=np.float32)
    L = np.empty((n,), dtype=np.float32)
    lib = lib or _load()
    if window is not None:
        rc = lib.fa_oracle_fwd_swa(_ptr(qf), _ptr(kf), _ptr(vf), _ptr(mf), B, H, Hkv, ql, kl,
                                   D, float(scale), int(window), rows.ctypes.data, n, _ptr(O),
                                   _ptr(L), n_threads or default_threads())
        _check(rc, "fa_oracle_fwd_swa")
        return O, round_bf16(O, lib), L
    rc = lib.fa_oracle_fwd_rows(_ptr(qf), _ptr(kf), _ptr(vf), _ptr(mf), B, H, Hkv, ql, kl,
                                    D, float(scale), int(bool(causal)), _ptr(rows), n, _ptr(O),
                                    _ptr(L), n_threads or default_threads())
    _check(rc, "fa_oracle_fwd_rows")
    return O, round_bf16(O, lib), L


def bwd(q, k, v, mask, L, dO, B, H, Hkv, ql, kl, D, scale, causal, n_threads=None,
        lib=None, window=None, O=None):
    """Backward (the page's FA-2 backward oracle). q/k/v/dO: bf16 bits or f32;
    mask f32 or None; L: the forward's natural-log logsumexp [B,H,ql];
    window: None or a sliding window (>= 0, with causal). O: None (D_i is
    sum_j P_ij dP_ij) or the O [B,H,ql,D] (bf16 bits or f32) that
    D_i = rowsum(O_i * dO_i) is read from.

    Returns (dQ [B,H,ql,D], dK [B,Hkv,kl,D], dV [B,Hkv,kl,D]), all f32."""
    qf, kf, vf, mf, lf, gf = _f32(q), _f32(k), _f32(v), _f32(mask), _f32(L), _f32(dO)
    dQ = np.empty((B, H, ql, D), dtype=np.float32)
    dK = np.empty((B, Hkv, kl, D), dtype=np.float32)
    dV = np.empty((B, Hkv, kl, D), dtype=np.float32)
    lib = lib or _load()
    if O is not None:
        of = _f32(O)
        if of.size != B * H * ql * D:
            raise ValueError(f"O must hold {B * H * ql * D} values")
        rc = lib.fa_oracle_bwd_given_o(_ptr(qf), _ptr(kf), _ptr(vf), _ptr(mf), _ptr(lf),
                                       _ptr(gf), _ptr(of), B, H, Hkv, ql, kl, D, D, float(scale),
                                       int(bool(causal)), -1 if window is None else int(window),
                                       _ptr(dQ), _ptr(dK), _ptr(dV),
                                       n_threads or default_threads())
        _check(rc, "fa_oracle_bwd_given_o")
    elif window is not None:
        rc = lib.fa_oracle_bwd_swa(_ptr(qf), _ptr(kf), _ptr(vf), _ptr(mf), _ptr(lf), _ptr(gf), B,
                                   H, Hkv, ql, kl, D, float(scale), int(bool(causal)),
                                   int(window), _ptr(dQ), _ptr(dK), _ptr(dV),
                                   n_threads or default_threads())
        _check(rc, "fa_oracle_bwd_swa")
    else:
        rc = lib.fa_oracle_bwd(_ptr(qf), _ptr(kf), _ptr(vf), _ptr(mf), _ptr(lf), _ptr(gf), B, H,
                               Hkv, ql, kl, D, float(scale), int(bool(causal)), _ptr(dQ),
                               _ptr(dK), _ptr(dV), n_threads or default_threads())
        _check(rc, "fa_oracle_bwd")
    if kl == 0:
        dQ[...] = 0.0
    return dQ, dK, dV


def bwd_sinks(q, k, v, mask, L, dO, B, H, Hkv, ql, kl, D, scale, causal, sinks, window=None,
              n_threads=None, lib=None):
    """The gradient of sum(O * dO) with respect to each query head's sink
    logit: dsink_h = -sum over (b, i) of exp(sink_h - L_i) * D_i, with D_i the
    backward's sum_j P_ij dP_ij. L: the forward's logsumexp with the same sinks.
    Returns dsinks [H], f32. (dQ, dK and dV with sinks are bwd() given that L.)"""
    qf, kf, vf, mf, lf, gf = _f32(q), _f32(k), _f32(v), _f32(mask), _f32(L), _f32(dO)
    sf = np.ascontiguousarray(sinks, dtype=np.float32)
    if sf.shape != (H,):
        raise ValueError(f"sinks must have shape ({H},)")
    out = np.empty(H, dtype=np.float32)
    lib = lib or _load()
    rc = lib.fa_oracle_bwd_sinks(_ptr(qf), _ptr(kf), _ptr(vf), _ptr(mf), _ptr(lf), _ptr(gf), B, H,
                                 Hkv, ql, kl, D, D, float(scale), int(bool(causal)),
                                 -1 if window is None else int(window), _ptr(sf), _ptr(out),
                                 n_threads or default_threads())
    _check(rc, "fa_oracle_bwd_sinks")
    return out


def fwd_dv(q, k, v, mask, B, H, Hkv, ql, kl, D, Dv, scale, causal, window=None, rows=None,
           n_threads=None, lib=None, sinks=None):
    """Forward with value width Dv (q, k: [.., D]; v: [B,Hkv,kl,Dv]). All rows
    (O [B,H,ql,Dv], L [B,H,ql]) or the flat `rows` (O [n,Dv], L [n]).
    sinks: None or one logit per query head (f32 [H], natural-log units).
    Returns (O_f32, O_bf16_bits, L)."""
    qf, kf, vf, mf = _f32(q), _f32(k), _f32(v), _f32(mask)
    sf = None if sinks is None else np.ascontiguousarray(sinks, dtype=np.float32)
    if sf is not None and sf.shape != (H,):
        raise ValueError(f"sinks must have shape ({H},)")
    lib = lib or _load()
    if rows is None:
        O = np.empty((B, H, ql, Dv), dtype=np.float32)
        L = np.empty((B, H, ql), dtype=np.float32)
        rp, n = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        O = np.empty((rows.size, Dv), dtype=np.float32)
        L = np.empty((rows.size,), dtype=np.float32)
        rp, n = rows.ctypes.data, rows.size
        if n == 0:
            return O, round_bf16(O, lib), L
    if sf is None:
        rc = lib.fa_oracle_fwd_general(_ptr(qf), _ptr(kf), _ptr(vf), _ptr(mf), B, H, Hkv, ql, kl,
                                       D, Dv, float(scale), int(bool(causal)),
                                       -1 if window is None else int(window), rp, n, _ptr(O),
                                       _ptr(L), n_threads or default_threads())
        _check(rc, "fa_oracle_fwd_general")
    else:
        rc = lib.fa_oracle_fwd_sinks(_ptr(qf), _ptr(kf), _ptr(vf), _ptr(mf), B, H, Hkv, ql, kl,
                                     D, Dv, float(scale), int(bool(causal)),
                                     -1 if window is None else int(window), _ptr(sf), rp, n,
                                     _ptr(O), _ptr(L), n_threads or default_threads())
        _check(rc, "fa_oracle_fwd_sinks")
    return O, round_bf16(O, lib), L


def bwd_groups(q, k, v, mask, L, dO, B, H, Hkv, ql, kl, D, scale, causal, groups, Dv=None,
               window=None, n_threads=None, lib=None):
    """Backward of the kv heads `groups` (flat b * Hkv + g) only. Returns
    (dQ [n, H/Hkv, ql, D] of each group's query heads, dK [n, kl, D],
    dV [n, kl, Dv]), f32."""
    Dv = D if Dv is None else Dv
    qf, kf, vf, mf, lf, gf = _f32(q), _f32(k), _f32(v), _f32(mask), _f32(L), _f32(dO)
    groups = np.ascontiguousarray(groups, dtype=np.int64)
    n, G = groups.size, H // Hkv
    dQ = np.empty((n, G, ql, D), dtype=np.float32)
    dK = np.empty((n, kl, D), dtype=np.float32)
    dV = np.empty((n, kl, Dv), dtype=np.float32)
    if n == 0:
        return dQ, dK, dV
    lib = lib or _load()
    rc = lib.fa_oracle_bwd_general(_ptr(qf), _ptr(kf), _ptr(vf), _ptr(mf), _ptr(lf), _ptr(gf), B,
                                   H, Hkv, ql, kl, D, Dv, float(scale), int(bool(causal)),
                                   -1 if window is None else int(window), groups.ctypes.data, n,
                                   _ptr(dQ), _ptr(dK), _ptr(dV), n_threads or default_threads())
    _check(rc, "fa_oracle_bwd_general")
    return dQ, dK, dV


def bind(lib_path):
    """A fwd(...) callable over another build of fa_oracle.c (used by the
    mutation tests, which plant mistakes in a copy of the source)."""
    lib = _bind(lib_path)

    def f(*args, **kw):
        return fwd(*args, lib=lib, **kw)
    return f


def bind_dv(lib_path):
    """A fwd_dv(...) callable over another build of fa_oracle.c (mutation tests)."""
    lib = _bind(lib_path)

    def f(*args, **kw):
        return fwd_dv(*args, lib=lib, **kw)
    return f


def bind_bwd(lib_path):
    """A bwd(...) callable over another build of fa_oracle.c (mutation tests)."""
    lib = _bind(lib_path)

    def f(*args, **kw):
        return bwd(*args, lib=lib, **kw)
    return f


def bind_bwd_sinks(lib_path):
    """A bwd_sinks(...) callable over another build of fa_oracle.c (mutation tests)."""
    lib = _bind(lib_path)

    def f(*args, **kw):
        return bwd_sinks(*args, lib=lib, **kw)
    return f


def fwd_workload(w, inputs, rows=None, n_threads=None, window=None):
    """Oracle on a fagen.Workload and its generated inputs (all rows, or `rows`)."""
    args = (inputs["q"], inputs["k"], inputs["v"], inputs["mask"],
            w.B, w.H, w.Hkv, w.ql, w.kl, w.D, w.scale, w.causal)
    if rows is None:
        return fwd(*args, n_threads=n_threads, window=window)
    return fwd_rows(*args, rows, n_threads=n_threads, window=window)
