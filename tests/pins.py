"""Pins for an oracle callable fwd(q, k, v, mask, B, H, Hkv, ql, kl, D, scale,
causal) -> (O_f32, O_bf16_bits, L).

Each pin checks the oracle against something other than its own code: the
double-precision textbook definition (tests/brute.py), closed forms, exact
special cases or invariances that the mathematics of softmax attention fixes.
They are functions (not tests) so that test_oracle_mutants.py can run them
against deliberately broken builds of the oracle.
"""
import math

import numpy as np

import fagen
from tests.brute import attention_f64


def _widen(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _bf16_bits(x):
    """Exact bf16 bit patterns of float32 values that are already bf16 numbers."""
    u = np.asarray(x, np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


def _inputs(seed, B, H, Hkv, ql, kl, D, sigma=1.0):
    q = fagen.normal_bf16(seed, 0, (B, H, ql, D), sigma)
    k = fagen.normal_bf16(seed, 1, (B, Hkv, kl, D), sigma)
    v = fagen.normal_bf16(seed, 2, (B, Hkv, kl, D), sigma)
    return q, k, v


def _finite_mask(seed, B, H, ql, kl, p=0.2):
    """-inf with probability p, one fully -inf row per (b,h) when ql > 1, and
    finite N(0, 2^2) values elsewhere (so the mask's scale matters)."""
    m, _ = fagen.mask_f32(seed, B, H, ql, kl, p, 1 if ql > 1 else 0)
    vals = _widen(fagen.normal_bf16(seed, 9, (B, H, ql, kl), 2.0)).reshape(B, H, ql, kl)
    return np.where(np.isneginf(m), -np.inf, vals).astype(np.float32)


def pin_brute_force(fwd, B, H, Hkv, ql, kl, D, causal, masked, seed, scale=None, window=None):
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q, k, v = _inputs(seed, B, H, Hkv, ql, kl, D)
    mask = _finite_mask(seed, B, H, ql, kl) if masked else None
    kw = {} if window is None else {"window": window}
    O, Ob, L = fwd(q, k, v, mask, B, H, Hkv, ql, kl, D, scale, causal, **kw)
    Oref, Lref = attention_f64(_widen(q), _widen(k), _widen(v), mask, scale, causal, window)
    empty = np.isneginf(Lref)
    assert np.array_equal(np.isneginf(L), empty), "fully masked rows differ"
    assert np.all(O[empty] == 0) and not np.signbit(O[empty]).any(), "empty row O != +0"
    if (~empty).any():
        live = ~empty
        errO = np.abs(O[live] - Oref[live]).max()
        errL = (np.abs(L[live] - Lref[live]) / np.maximum(1.0, np.abs(Lref[live]))).max()
        assert errO <= 1e-5, f"O vs f64 brute force: {errO:.3e}"
        assert errL <= 1e-5, f"L vs f64 brute force: {errL:.3e}"


def pin_hand_worked(fwd):
    """Two keys, D=2, scale 1: q=(1,0), k0=(1,0), k1=(0,1), v0=(1,2), v1=(3,4).
    Scores are (1, 0), so L = ln(1 + e) and O = (e*v0 + v1) / (1 + e).
    Causal with ql=kl=2: row 0 sees only key 0 (L = 1, O = v0); row 1 with
    q=(0,1) has scores (0, 1): L = ln(1 + e), O = (v0 + e*v1) / (1 + e)."""
    e = math.e
    q = _bf16_bits(np.array([1, 0], np.float32)).reshape(1, 1, 1, 2)
    k = _bf16_bits(np.array([1, 0, 0, 1], np.float32)).reshape(1, 1, 2, 2)
    v = _bf16_bits(np.array([1, 2, 3, 4], np.float32)).reshape(1, 1, 2, 2)
    O, _, L = fwd(q, k, v, None, 1, 1, 1, 1, 2, 2, 1.0, False)
    want = np.array([(e * 1 + 3) / (1 + e), (e * 2 + 4) / (1 + e)])
    assert abs(L[0, 0, 0] - math.log(1 + e)) < 1e-6
    assert np.abs(O[0, 0, 0] - want).max() < 1e-6
    q2 = _bf16_bits(np.array([1, 0, 0, 1], np.float32)).reshape(1, 1, 2, 2)
    O, _, L = fwd(q2, k, v, None, 1, 1, 1, 2, 2, 2, 1.0, True)
    assert abs(L[0, 0, 0] - 1.0) < 1e-6
    assert np.abs(O[0, 0, 0] - np.array([1.0, 2.0])).max() < 1e-6
    assert abs(L[0, 0, 1] - math.log(1 + e)) < 1e-6
    want1 = np.array([(1 + e * 3) / (1 + e), (2 + e * 4) / (1 + e)])
    assert np.abs(O[0, 0, 1] - want1).max() < 1e-6


def pin_zero_q(fwd, ql=8, kl=8, causal=False, D=16):
    """Q = 0: every visible score is 0, so L_i = ln(n_i) (n_i visible keys)
    and O_i is the plain mean of the visible V rows."""
    B, H, Hkv = 1, 2, 1
    _, k, v = _inputs(1234 + ql + kl, B, H, Hkv, ql, kl, D)
    q = np.zeros((B, H, ql, D), np.uint16)
    O, _, L = fwd(q, k, v, None, B, H, Hkv, ql, kl, D, 0.125, causal)
    vf = _widen(v).astype(np.float64)
    off = max(kl - ql, 0)
    for h in range(H):
        for i in range(ql):
            n = min(off + i + 1, kl) if causal else kl
            assert abs(L[0, h, i] - math.log(n)) <= 1e-6 * max(1.0, math.log(n)), (i, n)
            mean = vf[0, 0, :n].mean(axis=0)
            assert np.abs(O[0, h, i] - mean).max() <= 1e-5, (i, n)


def pin_constant_v(fwd):
    """Every key row of V equal to the same bf16 vector c: O = c exactly after
    rounding to bf16, whatever the weights (they sum to one)."""
    B, H, Hkv, ql, kl, D = 2, 4, 2, 12, 20, 16
    q, k, _ = _inputs(99, B, H, Hkv, ql, kl, D)
    c = fagen.normal_bf16(98, 3, (D,), 1.0)
    v = np.broadcast_to(c, (B, Hkv, kl, D)).copy()
    mask = _finite_mask(97, B, H, ql, kl, p=0.3)
    for causal in (False, True):
        for m in (None, mask):
            O, Ob, L = fwd(q, k, v, m, B, H, Hkv, ql, kl, D, 0.25, causal)
            live = np.isfinite(L)
            assert np.array_equal(Ob[live], np.broadcast_to(c, Ob.shape)[live])


def pin_fully_masked(fwd):
    """Rows whose additive mask is entirely -inf: O = +0 and L = -inf exactly;
    all other rows finite."""
    B, H, Hkv, ql, kl, D = 1, 2, 2, 6, 9, 8
    q, k, v = _inputs(5, B, H, Hkv, ql, kl, D)
    mask = np.zeros((B, H, ql, kl), np.float32)
    mask[0, 0, 2] = -np.inf
    mask[0, 1, 0] = -np.inf
    mask[0, 1, 5] = -np.inf
    for causal in (False, True):
        O, Ob, L = fwd(q, k, v, mask, B, H, Hkv, ql, kl, D, 0.3, causal)
        dead = np.isneginf(mask).all(-1)
        assert np.isneginf(L[dead]).all() and np.isfinite(L[~dead]).all()
        assert np.all(O[dead] == 0) and not np.signbit(O[dead]).any()
        assert np.all(Ob[dead] == 0)
        assert np.isfinite(O).all()


def pin_zero_mask(fwd):
    """An all-zero additive mask adds exactly 0 to every score: bit-identical."""
    B, H, Hkv, ql, kl, D = 1, 2, 1, 10, 14, 8
    q, k, v = _inputs(6, B, H, Hkv, ql, kl, D)
    zero = np.zeros((B, H, ql, kl), np.float32)
    for causal in (False, True):
        a = fwd(q, k, v, None, B, H, Hkv, ql, kl, D, 0.35, causal)
        b = fwd(q, k, v, zero, B, H, Hkv, ql, kl, D, 0.35, causal)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2])


def pin_mask_shift(fwd):
    """Adding a constant c_i to a whole mask row leaves softmax unchanged and
    shifts L_i by c_i."""
    B, H, Hkv, ql, kl, D = 1, 2, 2, 7, 11, 8
    q, k, v = _inputs(7, B, H, Hkv, ql, kl, D)
    mask = _finite_mask(8, B, H, ql, kl, p=0.2)
    shift = np.linspace(-3.0, 2.5, ql, dtype=np.float32)[None, None, :]
    O0, _, L0 = fwd(q, k, v, mask, B, H, Hkv, ql, kl, D, 0.4, False)
    O1, _, L1 = fwd(q, k, v, mask + shift[..., None], B, H, Hkv, ql, kl, D, 0.4, False)
    live = np.isfinite(L0)
    assert np.array_equal(live, np.isfinite(L1))
    assert np.abs(O1 - O0)[live].max() <= 1e-5
    dL = L1[live] - L0[live]
    assert np.abs(dL - np.broadcast_to(shift, L0.shape)[live]).max() <= 1e-5


def pin_causal_sentinel(fwd):
    """The method page's causal falsifier (section 6): K rows after a target
    query are set to 128.0, which would dominate any softmax that saw them.
    Under causal masking, O rows 0..target are bit-identical to the run on the
    clean K; without causal masking they change."""
    B, H, Hkv, ql, kl, D = 1, 1, 1, 32, 32, 64
    target = 15
    q, k, v = _inputs(40, B, H, Hkv, ql, kl, D)
    kp = k.copy()
    kp[0, 0, target + 1:] = _bf16_bits(np.array([128.0], np.float32))[0]
    a = fwd(q, k, v, None, B, H, Hkv, ql, kl, D, 0.125, True)
    b = fwd(q, kp, v, None, B, H, Hkv, ql, kl, D, 0.125, True)
    assert np.array_equal(a[0][0, 0, :target + 1], b[0][0, 0, :target + 1])
    assert np.array_equal(a[2][0, 0, :target + 1], b[2][0, 0, :target + 1])
    c = fwd(q, kp, v, None, B, H, Hkv, ql, kl, D, 0.125, False)
    d = fwd(q, k, v, None, B, H, Hkv, ql, kl, D, 0.125, False)
    assert not np.array_equal(c[0][0, 0, :target + 1], d[0][0, 0, :target + 1])


def pin_causal_alignment(fwd):
    """Key j is visible to row i iff j <= max(kl - ql, 0) + i: perturbing V row
    j changes exactly the rows with max(kl-ql,0) + i >= j, bit for bit. With
    Q = 0 every visible key has weight 1/n_i, so a visible change cannot hide
    below the rounding of O."""
    D = 8
    for ql, kl in [(5, 9), (9, 5), (6, 6)]:
        B, H, Hkv = 1, 1, 1
        _, k, v = _inputs(41 + ql, B, H, Hkv, ql, kl, D)
        q = np.zeros((B, H, ql, D), np.uint16)
        off = max(kl - ql, 0)
        base = fwd(q, k, v, None, B, H, Hkv, ql, kl, D, 0.5, True)[0]
        for j in range(kl):
            vp = v.copy()
            vp[0, 0, j] = _bf16_bits(np.array([7.0], np.float32))[0]
            out = fwd(q, k, vp, None, B, H, Hkv, ql, kl, D, 0.5, True)[0]
            for i in range(ql):
                changed = not np.array_equal(out[0, 0, i], base[0, 0, i])
                assert changed == (off + i >= j), (ql, kl, i, j)


def pin_gqa_repeat(fwd):
    """GQA with group g equals MHA with each K/V head repeated g times
    (consecutive query heads share a KV head): bit-identical."""
    B, H, Hkv, ql, kl, D = 2, 6, 2, 9, 13, 8
    q, k, v = _inputs(42, B, H, Hkv, ql, kl, D)
    g = H // Hkv
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    mask = _finite_mask(43, B, H, ql, kl)
    for causal in (False, True):
        a = fwd(q, k, v, mask, B, H, Hkv, ql, kl, D, 0.3, causal)
        b = fwd(q, kr, vr, mask, B, H, H, ql, kl, D, 0.3, causal)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2])


def pin_dominant_key(fwd):
    """One key whose score exceeds every other by far more than the f32 range
    of exp2 (about 290 in base 2): the softmax is one-hot on it, so O equals
    that V row and L equals its natural-log score. The dominant key is the
    last visible one, so a row max that skipped any key would overflow."""
    B, H, Hkv, ql, kl, D = 1, 1, 1, 4, 6, 8
    _, _, v = _inputs(44, B, H, Hkv, ql, kl, D)
    q = np.zeros((B, H, ql, D), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((B, Hkv, kl, D), np.float32)
    k[0, 0, :, 0] = np.array([0.5, -1.0, 0.25, 2.0, 1.5, 100.0], np.float32)
    scale = 2.0
    O, Ob, L = fwd(_bf16_bits(q), _bf16_bits(k), v, None, B, H, Hkv, ql, kl, D, scale, False)
    vb = np.asarray(v, np.uint16)
    for i in range(ql):
        assert np.array_equal(Ob[0, 0, i], vb[0, 0, kl - 1]), i
        assert abs(L[0, 0, i] - 200.0) <= 1e-4, L[0, 0, i]
    # causal with ql = kl: the dominant key is visible to the last row only,
    # where it is also the last visible key
    q6 = np.zeros((B, H, kl, D), np.float32)
    q6[..., 0] = 1.0
    O, Ob, L = fwd(_bf16_bits(q6), _bf16_bits(k), v, None, B, H, Hkv, kl, kl, D, scale, True)
    assert np.array_equal(Ob[0, 0, kl - 1], vb[0, 0, kl - 1])
    assert abs(L[0, 0, kl - 1] - 200.0) <= 1e-4
    assert np.isfinite(L).all() and np.isfinite(O).all()


def swa_mask(B, H, ql, kl, window):
    """The page's sliding-window additive mask (section 7): 0 where
    j <= q_abs and j + window >= q_abs, -inf elsewhere, with q_abs = i + the
    causal offset max(kl - ql, 0)."""
    off = max(kl - ql, 0)
    i = np.arange(ql)[:, None] + off
    j = np.arange(kl)[None, :]
    keep = (j <= i) & (j + window >= i)
    m = np.where(keep, 0.0, -np.inf).astype(np.float32)
    return np.broadcast_to(m, (B, H, ql, kl)).copy()


def pin_window_is_the_page_mask(fwd):
    """A native window gives bit-for-bit what the page's construction gives:
    the same predicate written into an additive 0/-inf mask, run without the
    causal flag (adding 0 leaves a score unchanged; -inf hides it)."""
    for (ql, kl, w) in [(20, 20, 5), (9, 23, 3), (23, 9, 4), (12, 12, 0), (7, 7, 30)]:
        B, H, Hkv, D = 1, 4, 2, 8
        q, k, v = _inputs(300 + ql + kl + w, B, H, Hkv, ql, kl, D)
        a = fwd(q, k, v, None, B, H, Hkv, ql, kl, D, 0.4, True, window=w)
        b = fwd(q, k, v, swa_mask(B, H, ql, kl, w), B, H, Hkv, ql, kl, D, 0.4, False)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2]), (ql, kl, w)


def pin_window_alignment(fwd):
    """Key j is visible to row i iff q_abs - w <= j <= q_abs: perturbing V row
    j changes exactly those rows, bit for bit (Q = 0, so every visible key
    weighs 1/n_i and no change can hide in rounding)."""
    D = 8
    for ql, kl, w in [(6, 10, 2), (10, 6, 3), (8, 8, 0), (8, 8, 4)]:
        B, H, Hkv = 1, 1, 1
        _, k, v = _inputs(51 + ql + w, B, H, Hkv, ql, kl, D)
        q = np.zeros((B, H, ql, D), np.uint16)
        off = max(kl - ql, 0)
        base = fwd(q, k, v, None, B, H, Hkv, ql, kl, D, 0.5, True, window=w)[0]
        for j in range(kl):
            vp = v.copy()
            vp[0, 0, j] = _bf16_bits(np.array([7.0], np.float32))[0]
            out = fwd(q, k, vp, None, B, H, Hkv, ql, kl, D, 0.5, True, window=w)[0]
            for i in range(ql):
                changed = not np.array_equal(out[0, 0, i], base[0, 0, i])
                assert changed == (off + i - w <= j <= off + i), (ql, kl, w, i, j)


def pin_window_zero(fwd):
    """window = 0: each row sees only key q_abs, so O is that V row exactly and
    L its natural-log score scale * q.k (rows with q_abs >= kl see nothing)."""
    B, H, Hkv, D = 1, 2, 1, 16
    for ql, kl in [(9, 9), (5, 11), (11, 5)]:
        q, k, v = _inputs(61 + ql, B, H, Hkv, ql, kl, D)
        O, Ob, L = fwd(q, k, v, None, B, H, Hkv, ql, kl, D, 0.25, True, window=0)
        off = max(kl - ql, 0)
        qf, kf = _widen(q).astype(np.float64), _widen(k).astype(np.float64)
        for h in range(H):
            for i in range(ql):
                j = off + i
                if j >= kl:
                    assert np.isneginf(L[0, h, i]) and np.all(O[0, h, i] == 0)
                    continue
                assert np.array_equal(Ob[0, h, i], v[0, 0, j]), (h, i)
                s = 0.25 * float(qf[0, h, i] @ kf[0, 0, j])
                assert abs(L[0, h, i] - s) <= 1e-5 * max(1.0, abs(s)), (h, i, L[0, h, i], s)


def pin_window_wide_is_causal(fwd):
    """A window at least as wide as every row's visible range hides nothing the
    causal rule leaves visible: bit-identical to the causal forward."""
    B, H, Hkv, ql, kl, D = 2, 2, 1, 10, 14, 8
    q, k, v = _inputs(71, B, H, Hkv, ql, kl, D)
    mask = _finite_mask(72, B, H, ql, kl)
    for w in (kl - 1, kl, 10 * kl):
        a = fwd(q, k, v, mask, B, H, Hkv, ql, kl, D, 0.3, True, window=w)
        b = fwd(q, k, v, mask, B, H, Hkv, ql, kl, D, 0.3, True)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2]), w


def pin_brute_force_dv(fwd_dv, B, H, Hkv, ql, kl, D, Dv, causal, masked, seed, window=None):
    """Values wider or narrower than the keys (Dv != D) against the f64
    textbook definition; fwd_dv(q, k, v, mask, B, H, Hkv, ql, kl, D, Dv,
    scale, causal, window=...) -> (O [B,H,ql,Dv], O bits, L)."""
    scale = 1.0 / math.sqrt(D)
    q = fagen.normal_bf16(seed, 0, (B, H, ql, D))
    k = fagen.normal_bf16(seed, 1, (B, Hkv, kl, D))
    v = fagen.normal_bf16(seed, 2, (B, Hkv, kl, Dv))
    mask = _finite_mask(seed, B, H, ql, kl) if masked else None
    O, Ob, L = fwd_dv(q, k, v, mask, B, H, Hkv, ql, kl, D, Dv, scale, causal, window=window)
    assert O.shape == (B, H, ql, Dv)
    Oref, Lref = attention_f64(_widen(q), _widen(k), _widen(v), mask, scale, causal, window)
    empty = np.isneginf(Lref)
    assert np.array_equal(np.isneginf(L), empty), "fully masked rows differ"
    assert np.all(O[empty] == 0), "empty row O != 0"
    live = ~empty
    if live.any():
        errO = np.abs(O[live] - Oref[live]).max()
        errL = (np.abs(L[live] - Lref[live]) / np.maximum(1.0, np.abs(Lref[live]))).max()
        assert errO <= 1e-5, f"O (Dv={Dv}) vs f64 brute force: {errO:.3e}"
        assert errL <= 1e-5, f"L (Dv={Dv}) vs f64 brute force: {errL:.3e}"


# Pins of the forward with a separate value width (fwd_dv callables).
DV_PINS = [
    ("brute_dv_wide", lambda f: pin_brute_force_dv(f, 2, 4, 2, 9, 13, 8, 24, True, True, 5)),
    ("brute_dv_narrow", lambda f: pin_brute_force_dv(f, 1, 2, 1, 11, 7, 24, 8, False, False, 6)),
    ("brute_dv_window", lambda f: pin_brute_force_dv(f, 1, 2, 2, 12, 12, 16, 8, True, False, 7,
                                                     window=3)),
]

def pin_brute_force_sinks(fwd_dv, B, H, Hkv, ql, kl, D, Dv, causal, masked, seed, sinks):
    """Per-head sink logits against the f64 definition (one more softmax term
    with a zero value); fwd_dv as for pin_brute_force_dv, with sinks=."""
    scale = 1.0 / math.sqrt(D)
    q = fagen.normal_bf16(seed, 0, (B, H, ql, D))
    k = fagen.normal_bf16(seed, 1, (B, Hkv, kl, D))
    v = fagen.normal_bf16(seed, 2, (B, Hkv, kl, Dv))
    mask = _finite_mask(seed, B, H, ql, kl) if masked else None
    sinks = np.asarray(sinks, dtype=np.float32)
    O, _, L = fwd_dv(q, k, v, mask, B, H, Hkv, ql, kl, D, Dv, scale, causal, sinks=sinks)
    Oref, Lref = attention_f64(_widen(q), _widen(k), _widen(v), mask, scale, causal,
                               sinks=sinks)
    empty = np.isneginf(Lref)
    assert np.array_equal(np.isneginf(L), empty), "rows with L = -inf differ"
    assert np.all(O[empty] == 0), "empty row O != 0"
    live = ~empty
    errO = np.abs(O[live] - Oref[live]).max()
    errL = (np.abs(L[live] - Lref[live]) / np.maximum(1.0, np.abs(Lref[live]))).max()
    assert errO <= 1e-5, f"O with sinks vs f64 brute force: {errO:.3e}"
    assert errL <= 1e-5, f"L with sinks vs f64 brute force: {errL:.3e}"


def pin_sinks_closed_forms(fwd_dv):
    """What the definition fixes exactly: sinks of -inf change nothing (bit for
    bit); a row with no visible key gets O = +0 and L = its head's sink; a sink
    far above every score takes all the weight (O -> 0, L -> sink); and with a
    sink s, L' = logaddexp(L, s) and O' = O exp(L - L') for the row's no-sink
    L and O."""
    B, H, Hkv, ql, kl, D = 1, 4, 2, 6, 9, 8
    q, k, v = _inputs(11, B, H, Hkv, ql, kl, D)
    scale = 0.4
    O0, _, L0 = fwd_dv(q, k, v, None, B, H, Hkv, ql, kl, D, D, scale, True)
    neg = np.full(H, -np.inf, dtype=np.float32)
    On, _, Ln = fwd_dv(q, k, v, None, B, H, Hkv, ql, kl, D, D, scale, True, sinks=neg)
    assert np.array_equal(On, O0) and np.array_equal(Ln, L0), "sinks of -inf changed the result"
    s = np.array([-2.0, 0.5, 3.0, 1.25], dtype=np.float32)
    O1, _, L1 = fwd_dv(q, k, v, None, B, H, Hkv, ql, kl, D, D, scale, True, sinks=s)
    Lx = np.logaddexp(L0.astype(np.float64), s[None, :, None].astype(np.float64))
    assert np.abs(L1 - Lx).max() <= 1e-5 * max(1.0, np.abs(Lx).max()), "L != logaddexp(L, sink)"
    Ox = O0 * np.exp(L0.astype(np.float64) - Lx)[..., None]
    assert np.abs(O1 - Ox).max() <= 1e-5, "O != O exp(L - L')"
    big = np.full(H, 120.0, dtype=np.float32)
    Ob, _, Lb = fwd_dv(q, k, v, None, B, H, Hkv, ql, kl, D, D, scale, True, sinks=big)
    assert np.all(np.isfinite(Lb)) and np.abs(Lb - 120.0).max() <= 1e-4, "a dominant sink"
    assert np.abs(Ob).max() <= 1e-30, "a dominant sink leaves no weight to the keys"
    mask = np.zeros((B, H, ql, kl), dtype=np.float32)
    mask[:, :, 2] = -np.inf  # row 2 of every head sees no key
    Om, _, Lm = fwd_dv(q, k, v, mask, B, H, Hkv, ql, kl, D, D, scale, True, sinks=s)
    assert np.all(Lm[0, :, 2] == s), "an empty row's L must be its head's sink"
    assert np.all(_bf16_bits(Om[0, :, 2]) == 0) and not np.signbit(Om[0, :, 2]).any(), \
        "an empty row's O must be +0"


# Pins of the forward with sinks (fwd_dv callables taking sinks=).
SINK_PINS = [
    ("sinks_closed_forms", pin_sinks_closed_forms),
    ("brute_sinks", lambda f: pin_brute_force_sinks(f, 2, 4, 2, 9, 13, 8, 8, True, True, 8,
                                                    [-1.0, 0.0, 2.5, -np.inf])),
    ("brute_sinks_dv", lambda f: pin_brute_force_sinks(f, 1, 2, 1, 7, 5, 16, 8, False, False, 9,
                                                       [1.5, -0.5])),
]

ALL_PINS = [
    ("hand_worked", pin_hand_worked),
    ("brute_small", lambda f: pin_brute_force(f, 2, 4, 2, 9, 13, 8, True, True, 1)),
    ("brute_nocausal", lambda f: pin_brute_force(f, 1, 2, 1, 7, 5, 8, False, False, 2)),
    ("brute_offset", lambda f: pin_brute_force(f, 1, 2, 2, 5, 11, 16, True, False, 3)),
    ("zero_q", lambda f: pin_zero_q(f, 6, 9, True)),
    ("constant_v", pin_constant_v),
    ("fully_masked", pin_fully_masked),
    ("zero_mask", pin_zero_mask),
    ("mask_shift", pin_mask_shift),
    ("causal_sentinel", pin_causal_sentinel),
    ("causal_alignment", pin_causal_alignment),
    ("gqa_repeat", pin_gqa_repeat),
    ("dominant_key", pin_dominant_key),
    ("window_brute", lambda f: pin_brute_force(f, 2, 4, 2, 13, 17, 8, True, True, 4, window=5)),
    ("window_page_mask", pin_window_is_the_page_mask),
    ("window_alignment", pin_window_alignment),
    ("window_zero", pin_window_zero),
    ("window_wide", pin_window_wide_is_causal),
]
