"""Pins for a backward oracle callable bwd(q, k, v, mask, L, dO, B, H, Hkv,
ql, kl, D, scale, causal) -> (dQ, dK, dV).

Each pin checks the backward against something other than its own code:
torch's float64 autograd of the textbook definition (tests/brute.py), central
finite differences of the float64 forward, closed forms (constant V rows give
dQ = dK = 0; zero dO gives zero gradients) and the GQA invariance. L is taken
from the float64 forward, so these pins do not lean on the forward oracle.
Functions, not tests, so that test_oracle_mutants.py can run them against
deliberately broken builds of the oracle.
"""
import math

import numpy as np

import fagen
from tests.brute import attention_f64, attention_grads_f64
from tests.pins import _finite_mask, _inputs, _widen


def _case(seed, B, H, Hkv, ql, kl, D, masked):
    q, k, v = _inputs(seed, B, H, Hkv, ql, kl, D)
    dO = fagen.normal_bf16(seed, 7, (B, H, ql, D), 1.0)
    mask = _finite_mask(seed, B, H, ql, kl) if masked else None
    return q, k, v, dO, mask


def _lse(q, k, v, mask, scale, causal, window=None):
    _, L = attention_f64(_widen(q), _widen(k), _widen(v), mask, scale, causal, window)
    return L.astype(np.float32)


def pin_bwd_autograd(bwd, B, H, Hkv, ql, kl, D, causal, masked, seed, scale=None):
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q, k, v, dO, mask = _case(seed, B, H, Hkv, ql, kl, D, masked)
    L = _lse(q, k, v, mask, scale, causal)
    got = bwd(q, k, v, mask, L, dO, B, H, Hkv, ql, kl, D, scale, causal)
    ref = attention_grads_f64(_widen(q).reshape(B, H, ql, D), _widen(k).reshape(B, Hkv, kl, D),
                              _widen(v).reshape(B, Hkv, kl, D), mask,
                              _widen(dO).reshape(B, H, ql, D), scale, causal)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        err = np.abs(g - r).max() if r.size else 0.0
        tol = 2e-5 * max(1.0, np.abs(r).max() if r.size else 1.0)
        assert err <= tol, f"{name} vs f64 autograd: {err:.3e} > {tol:.3e}"


def pin_bwd_finite_difference(bwd, seed=31):
    """Central differences of sum(O * dO) of the float64 forward, at a few
    entries of Q, K and V (the page's falsifier, at more than one entry)."""
    B, H, Hkv, ql, kl, D, scale = 1, 2, 1, 6, 9, 8, 0.4
    q, k, v, dO, _ = _case(seed, B, H, Hkv, ql, kl, D, False)
    qf, kf, vf, gf = (_widen(x).astype(np.float64) for x in (q, k, v, dO))
    qf, gf = qf.reshape(B, H, ql, D), gf.reshape(B, H, ql, D)
    kf, vf = kf.reshape(B, Hkv, kl, D), vf.reshape(B, Hkv, kl, D)
    L = _lse(q, k, v, None, scale, True)
    dQ, dK, dV = bwd(q, k, v, None, L, dO, B, H, Hkv, ql, kl, D, scale, True)
    loss = lambda a, b_, c: float((attention_f64(a, b_, c, None, scale, True)[0] * gf).sum())
    h = 1e-4
    rng = np.random.default_rng(seed)
    for which, grad in (("q", dQ), ("k", dK), ("v", dV)):
        base = {"q": qf, "k": kf, "v": vf}[which]
        for _ in range(4):
            ix = tuple(int(rng.integers(0, n)) for n in base.shape)
            plus, minus = base.copy(), base.copy()
            plus[ix] += h
            minus[ix] -= h
            args_p = [qf, kf, vf]
            args_m = [qf, kf, vf]
            pos = "qkv".index(which)
            args_p[pos], args_m[pos] = plus, minus
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[ix]) <= 1e-4 * max(1.0, abs(fd)), \
                f"d{which.upper()}{ix}: finite difference {fd:.6f}, oracle {grad[ix]:.6f}"


def pin_bwd_constant_v(bwd):
    """Every V row equal to one vector c: dP_ij = dO_i . c is the same for all j,
    so dS = P (dP - D) = 0 and dQ = dK = 0; dV_j = sum_i P_ij dO_i."""
    B, H, Hkv, ql, kl, D, scale = 1, 2, 2, 7, 11, 16, 0.35
    q, k, _, dO, _ = _case(41, B, H, Hkv, ql, kl, D, False)
    c = fagen.normal_bf16(41, 5, (D,), 1.0)
    v = np.tile(c, B * Hkv * kl).reshape(B, Hkv, kl, D)
    L = _lse(q, k, v, None, scale, True)
    dQ, dK, dV = bwd(q, k, v, None, L, dO, B, H, Hkv, ql, kl, D, scale, True)
    assert np.abs(dQ).max() <= 2e-6 and np.abs(dK).max() <= 2e-6, "constant V: dQ, dK not 0"
    _, _, dVr = attention_grads_f64(_widen(q).reshape(B, H, ql, D), _widen(k).reshape(B, Hkv, kl, D),
                                    _widen(v).reshape(B, Hkv, kl, D), None,
                                    _widen(dO).reshape(B, H, ql, D), scale, True)
    assert np.abs(dV - dVr).max() <= 1e-5 * max(1.0, np.abs(dVr).max())


def pin_bwd_zero_do(bwd):
    B, H, Hkv, ql, kl, D, scale = 1, 2, 1, 5, 6, 8, 0.5
    q, k, v, _, mask = _case(43, B, H, Hkv, ql, kl, D, True)
    dO = np.zeros((B, H, ql, D), np.uint16)
    L = _lse(q, k, v, mask, scale, False)
    for g in bwd(q, k, v, mask, L, dO, B, H, Hkv, ql, kl, D, scale, False):
        assert np.all(g == 0), "zero upstream gradient must give zero gradients"


def pin_bwd_gqa(bwd):
    """Hkv < H equals the same problem with every query head given its own
    copy of its kv head, and dK, dV summed over each group."""
    B, H, Hkv, ql, kl, D, scale = 2, 4, 2, 6, 7, 8, 0.3
    q, k, v, dO, mask = _case(47, B, H, Hkv, ql, kl, D, True)
    L = _lse(q, k, v, mask, scale, True)
    dQ, dK, dV = bwd(q, k, v, mask, L, dO, B, H, Hkv, ql, kl, D, scale, True)
    rep = lambda a: np.repeat(a.reshape(B, Hkv, kl, D), H // Hkv, axis=1)
    dQ2, dK2, dV2 = bwd(q, rep(k), rep(v), mask, L, dO, B, H, H, ql, kl, D, scale, True)
    fold = lambda a: a.reshape(B, Hkv, H // Hkv, kl, D).sum(axis=2)
    assert np.abs(dQ - dQ2).max() <= 1e-6 * max(1.0, np.abs(dQ).max())
    assert np.abs(dK - fold(dK2)).max() <= 1e-5 * max(1.0, np.abs(dK).max())
    assert np.abs(dV - fold(dV2)).max() <= 1e-5 * max(1.0, np.abs(dV).max())


def pin_bwd_window_autograd(bwd, B, H, Hkv, ql, kl, D, window, masked, seed):
    """The sliding-window backward against float64 autograd of the textbook
    definition restricted to the band q_abs - w <= j <= q_abs."""
    scale = 1.0 / math.sqrt(D)
    q, k, v, dO, mask = _case(seed, B, H, Hkv, ql, kl, D, masked)
    L = _lse(q, k, v, mask, scale, True, window)
    got = bwd(q, k, v, mask, L, dO, B, H, Hkv, ql, kl, D, scale, True, window=window)
    ref = attention_grads_f64(_widen(q).reshape(B, H, ql, D), _widen(k).reshape(B, Hkv, kl, D),
                              _widen(v).reshape(B, Hkv, kl, D), mask,
                              _widen(dO).reshape(B, H, ql, D), scale, True, window)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        err = np.abs(g - r).max() if r.size else 0.0
        tol = 2e-5 * max(1.0, np.abs(r).max() if r.size else 1.0)
        assert err <= tol, f"{name} vs f64 autograd (window {window}): {err:.3e} > {tol:.3e}"


def pin_bwd_window_is_the_page_mask(bwd):
    """A native window gives the bits of the page's own construction, the
    0/-inf band mask run without the causal flag."""
    from tests.pins import swa_mask
    for (ql, kl, w) in [(12, 12, 3), (7, 15, 2), (15, 7, 4)]:
        B, H, Hkv, D, scale = 1, 2, 1, 8, 0.4
        q, k, v, dO, _ = _case(200 + ql + w, B, H, Hkv, ql, kl, D, False)
        L = _lse(q, k, v, None, scale, True, w)
        a = bwd(q, k, v, None, L, dO, B, H, Hkv, ql, kl, D, scale, True, window=w)
        b = bwd(q, k, v, swa_mask(B, H, ql, kl, w), L, dO, B, H, Hkv, ql, kl, D, scale, False)
        for x, y in zip(a, b):
            assert np.array_equal(x, y), (ql, kl, w)


def _lse_sinks(q, k, v, mask, scale, causal, sinks):
    _, L = attention_f64(_widen(q), _widen(k), _widen(v), mask, scale, causal, sinks=sinks)
    return L.astype(np.float32)


def pin_bwd_sinks_autograd(bwd, bwd_sinks, B, H, Hkv, ql, kl, D, causal, mask_kind, seed,
                           sinks):
    """With per-head sinks (one more softmax term with a zero value), dQ, dK and
    dV from the sink-aware L, and each sink's own gradient, against float64
    autograd of the textbook definition. mask_kind: None, "finite", or "rows"
    (some rows with no visible key, which keep only the sink)."""
    scale = 1.0 / math.sqrt(D)
    q, k, v, dO, mask = _case(seed, B, H, Hkv, ql, kl, D, mask_kind == "finite")
    if mask_kind == "rows":
        mask, _ = fagen.mask_f32(seed, B, H, ql, kl, 0.1, 2)
    sinks = np.asarray(sinks, dtype=np.float32)
    L = _lse_sinks(q, k, v, mask, scale, causal, sinks)
    got = list(bwd(q, k, v, mask, L, dO, B, H, Hkv, ql, kl, D, scale, causal))
    got.append(bwd_sinks(q, k, v, mask, L, dO, B, H, Hkv, ql, kl, D, scale, causal, sinks))
    ref = attention_grads_f64(_widen(q).reshape(B, H, ql, D), _widen(k).reshape(B, Hkv, kl, D),
                              _widen(v).reshape(B, Hkv, kl, D), mask,
                              _widen(dO).reshape(B, H, ql, D), scale, causal, sinks=sinks)
    for name, g, r in zip(("dQ", "dK", "dV", "dsinks"), got, ref):
        err = np.abs(g - r).max() if r.size else 0.0
        tol = 2e-5 * max(1.0, np.abs(r).max() if r.size else 1.0)
        assert err <= tol, f"{name} with sinks vs f64 autograd: {err:.3e} > {tol:.3e}"


def pin_bwd_sinks_finite_difference(bwd, bwd_sinks, seed=53):
    """Central differences of sum(O * dO) of the float64 forward in each sink."""
    B, H, Hkv, ql, kl, D, scale = 2, 3, 1, 6, 9, 8, 0.4
    q, k, v, dO, _ = _case(seed, B, H, Hkv, ql, kl, D, False)
    sinks = np.array([0.7, -1.3, 2.1], np.float32)
    L = _lse_sinks(q, k, v, None, scale, True, sinks)
    ds = bwd_sinks(q, k, v, None, L, dO, B, H, Hkv, ql, kl, D, scale, True, sinks)
    qf, kf, vf, gf = (_widen(x).astype(np.float64) for x in (q, k, v, dO))
    qf, gf = qf.reshape(B, H, ql, D), gf.reshape(B, H, ql, D)
    kf, vf = kf.reshape(B, Hkv, kl, D), vf.reshape(B, Hkv, kl, D)
    loss = lambda s: float((attention_f64(qf, kf, vf, None, scale, True, sinks=s)[0] * gf).sum())
    h = 1e-4
    for i in range(H):
        plus, minus = sinks.astype(np.float64), sinks.astype(np.float64)
        plus[i] += h
        minus[i] -= h
        fd = (loss(plus) - loss(minus)) / (2 * h)
        assert abs(fd - ds[i]) <= 1e-4 * max(1.0, abs(fd)), \
            f"dsink[{i}]: finite difference {fd:.6f}, oracle {ds[i]:.6f}"


def pin_bwd_sinks_closed_forms(bwd, bwd_sinks):
    """Sinks of -inf get exactly zero gradient; with every V row equal to one
    vector c, O_i = (1 - p_i) c with p_i = exp(sink_h - L_i), so
    dsink_h = -sum_i p_i (1 - p_i) <dO_i, c>."""
    B, H, Hkv, ql, kl, D, scale = 1, 2, 1, 7, 11, 16, 0.35
    q, k, _, dO, _ = _case(59, B, H, Hkv, ql, kl, D, False)
    c = fagen.normal_bf16(59, 5, (D,), 1.0)
    v = np.tile(c, B * Hkv * kl).reshape(B, Hkv, kl, D)
    neg = np.full(H, -np.inf, np.float32)
    L0 = _lse(q, k, v, None, scale, True)
    assert np.all(bwd_sinks(q, k, v, None, L0, dO, B, H, Hkv, ql, kl, D, scale, True, neg) == 0)
    sinks = np.array([1.5, -0.5], np.float32)
    L = _lse_sinks(q, k, v, None, scale, True, sinks)
    ds = bwd_sinks(q, k, v, None, L, dO, B, H, Hkv, ql, kl, D, scale, True, sinks)
    Lf = L.astype(np.float64).reshape(B, H, ql)
    gc = (_widen(dO).astype(np.float64).reshape(B, H, ql, D) @ _widen(c).astype(np.float64))
    p = np.exp(sinks.astype(np.float64)[None, :, None] - Lf)
    want = -(p * (1 - p) * gc).sum(axis=(0, 2))
    assert np.abs(ds - want).max() <= 2e-5 * max(1.0, np.abs(want).max()), (ds, want)


SINK_PINS = [
    ("sinks_autograd", lambda b, s: pin_bwd_sinks_autograd(b, s, 2, 4, 2, 7, 13, 16, True, None, 61,
                                                           [0.4, -2.0, 1.1, 3.0])),
    ("sinks_autograd_masked", lambda b, s: pin_bwd_sinks_autograd(b, s, 1, 2, 2, 9, 6, 8, False,
                                                                  "finite", 62, [-0.3, 0.9])),
    ("sinks_autograd_empty_rows", lambda b, s: pin_bwd_sinks_autograd(b, s, 2, 2, 1, 8, 10, 8,
                                                                      True, "rows", 63,
                                                                      [0.5, -np.inf])),
    ("sinks_finite_difference", pin_bwd_sinks_finite_difference),
    ("sinks_closed_forms", pin_bwd_sinks_closed_forms),
]



def pin_bwd_given_o_autograd(bwd, B, H, Hkv, ql, kl, D, causal, masked, seed, window=None):
    """D_i read from a given O: handed the float64 forward's O (as f32), the
    gradients equal float64 autograd of the textbook definition, for every
    row of every head (an O row of the wrong row or head would not)."""
    scale = 1.0 / math.sqrt(D)
    q, k, v, dO, mask = _case(seed, B, H, Hkv, ql, kl, D, masked)
    O, L = attention_f64(_widen(q), _widen(k), _widen(v), mask, scale, causal, window)
    got = bwd(q, k, v, mask, L.astype(np.float32), dO, B, H, Hkv, ql, kl, D, scale, causal,
              window=window, O=O.astype(np.float32))
    ref = attention_grads_f64(_widen(q).reshape(B, H, ql, D), _widen(k).reshape(B, Hkv, kl, D),
                              _widen(v).reshape(B, Hkv, kl, D), mask,
                              _widen(dO).reshape(B, H, ql, D), scale, causal, window)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        err = np.abs(g - r).max() if r.size else 0.0
        tol = 2e-5 * max(1.0, np.abs(r).max() if r.size else 1.0)
        assert err <= tol, f"{name} (given O) vs f64 autograd: {err:.3e} > {tol:.3e}"


def pin_bwd_given_o_single_key(bwd):
    """One key (kl = 1): P_i0 = 1 on every row that sees it, so with a given
    O' the closed forms are dQ_i = scale (dO_i.v_0 - O'_i.dO_i) k_0,
    dK_0 = scale sum_i (dO_i.v_0 - O'_i.dO_i) q_i over the group's rows and
    dV_0 = sum_i dO_i; a row whose key is masked (P = 0) gives dQ_i = 0 and
    adds nothing, whatever O'_i holds."""
    B, H, Hkv, ql, kl, D, scale = 1, 2, 1, 5, 1, 8, 0.35
    q, k, v, dO, _ = _case(71, B, H, Hkv, ql, kl, D, False)
    qf, gf = (_widen(x).astype(np.float64).reshape(B, H, ql, D) for x in (q, dO))
    k0, v0 = (_widen(x).astype(np.float64).reshape(D) for x in (k, v))
    mask = np.zeros((B, H, ql, kl), np.float32)
    mask[0, 1, 2, 0] = -np.inf
    live = np.isfinite(mask[..., 0])
    delta = np.random.default_rng(72).normal(0.0, 0.05, (B, H, ql, D))
    Op = np.where(live[..., None], v0 + delta, 3.0 + delta)
    L = np.where(live, scale * (qf @ k0), -np.inf).astype(np.float32)
    dQ, dK, dV = bwd(q, k, v, mask, L, dO, B, H, Hkv, ql, kl, D, scale, False,
                     O=Op.astype(np.float32))
    c = np.where(live, gf @ v0 - (Op.astype(np.float32).astype(np.float64) * gf).sum(-1), 0.0)
    want_dq = scale * c[..., None] * k0
    want_dk = scale * (c[..., None] * qf).sum(axis=(1, 2))
    want_dv = (live[..., None] * gf).sum(axis=(1, 2))
    for name, g, w in (("dQ", dQ, want_dq), ("dK", dK.reshape(B, D), want_dk),
                       ("dV", dV.reshape(B, D), want_dv)):
        tol = 2e-5 * max(1.0, np.abs(w).max())
        assert np.abs(g.reshape(w.shape) - w).max() <= tol, f"{name} (given O, one key)"
    assert np.all(dQ[0, 1, 2] == 0.0)


GIVEN_O_PINS = [
    ("given_o_autograd", lambda f: pin_bwd_given_o_autograd(f, 2, 4, 2, 7, 13, 16, True, True,
                                                            81)),
    ("given_o_autograd_ql_gt_kl", lambda f: pin_bwd_given_o_autograd(f, 1, 2, 1, 12, 5, 8, True,
                                                                     False, 82)),
    ("given_o_autograd_window", lambda f: pin_bwd_given_o_autograd(f, 1, 2, 2, 9, 17, 16, True,
                                                                   False, 83, window=3)),
    ("given_o_single_key", pin_bwd_given_o_single_key),
]


AUTOGRAD_CASES = [
    # B, H, Hkv, ql, kl, D, causal, masked, seed
    (1, 1, 1, 1, 1, 4, False, False, 1),
    (1, 2, 2, 5, 7, 8, False, False, 2),
    (1, 2, 1, 9, 9, 8, True, False, 3),
    (2, 4, 2, 7, 13, 16, True, True, 4),
    (1, 4, 1, 12, 5, 8, True, False, 5),    # ql > kl: offset clamped at 0
    (1, 2, 2, 17, 33, 64, True, True, 6),
    (1, 1, 1, 8, 8, 64, False, True, 7),
]

ALL_PINS = [(f"autograd{c}", (lambda c: lambda f: pin_bwd_autograd(f, *c))(c))
            for c in AUTOGRAD_CASES] + [
    ("finite_difference", pin_bwd_finite_difference),
    ("constant_v", pin_bwd_constant_v),
    ("zero_do", pin_bwd_zero_do),
    ("gqa", pin_bwd_gqa),
    ("window_autograd", lambda f: pin_bwd_window_autograd(f, 2, 4, 2, 13, 13, 8, 4, True, 8)),
    ("window_autograd_offset", lambda f: pin_bwd_window_autograd(f, 1, 2, 1, 9, 17, 16, 3, False,
                                                                 9)),
    ("window_autograd_ql_gt_kl", lambda f: pin_bwd_window_autograd(f, 1, 2, 2, 14, 6, 8, 2, False,
                                                                   10)),
    ("window_page_mask", pin_bwd_window_is_the_page_mask),
]
