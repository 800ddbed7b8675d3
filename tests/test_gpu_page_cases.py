"""The method page's own test cases, on its own inputs, at its own bounds.

"mlx-native 0.9.0", tests/test_flash_attn_train.rs: the forward tests of
sections 2-8 and the backward tests of sections 11-16, each with the shapes,
causal flags, masks and seeds printed there. Inputs come from the page's
64-bit LCG (section "Test helpers", pseudo_random_f32, seeds SEED_VAL + k;
fagen.lcg_*), rounded to bf16. The HIP library runs them through the C ABI;
the oracle is the CPU reference. Bounds are the page's: O within 5e-3 of the
oracle's O rounded to bf16, L within 3e-3, dQ, dK and dV within 5e-3 of the
oracle's f32 gradients (computed, as on the page, from the oracle's own L);
the finite-difference falsifier of section 13 within 5e-2.
"""
import math

import numpy as np
import pytest

import fagen
import oracle
import flash_attention_forward_fa_amd as fa
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SEED = fagen.SEED_BASE  # the page's SEED_VAL ("TRAIN001")


def _dev(bits):
    return gu.to_dev(bits, "cuda:0")


def _swa_mask_bf16(B, H, ql, kl, window):
    """The page's sliding-window mask (sections 7 and 15): 0 where j <= i and
    j + window >= i, -inf elsewhere, as bf16 bits."""
    i = np.arange(ql)[:, None]
    j = np.arange(kl)[None, :]
    keep = (j <= i) & (j + window >= i)
    m = np.where(keep, np.float32(0.0), np.float32(-np.inf)).astype(np.float32)
    bits = (np.broadcast_to(m, (B, H, ql, kl)).copy().view(np.uint32) >> 16).astype(np.uint16)
    return bits


def _forward(q, k, v, mask_bits, B, H, Hkv, ql, kl, D, causal):
    import torch
    mask = None
    if mask_bits is not None:
        mask = _dev(mask_bits)  # bf16, as the page passes it
    O, L = fa.train_fwd_ex(_dev(q), _dev(k), _dev(v), mask=mask, scale=1.0 / math.sqrt(D),
                           causal=causal)
    torch.cuda.synchronize()
    bits = O.view(torch.int16).cpu().numpy().view(np.uint16)
    return gu.widen(bits), L.cpu().numpy(), bits


FWD_CASES = [
    # (section, B, H, Hkv, ql, kl, D, causal, window, seed offset, checks)
    ("2 O parity D=64", 1, 1, 1, 32, 32, 64, False, None, 0, "O"),
    ("3 L parity D=64", 1, 1, 1, 32, 32, 64, False, None, 10, "L"),
    ("4 O and L D=256", 1, 4, 4, 128, 128, 256, False, None, 20, "OL"),
    ("5 causal", 1, 2, 2, 64, 64, 64, True, None, 30, "OL"),
    ("7 sliding window mask", 1, 2, 2, 64, 64, 64, False, 16, 50, "OL"),
    ("8 GQA", 1, 8, 2, 64, 64, 64, False, None, 60, "OL"),
]


@pytest.mark.parametrize("sec,B,H,Hkv,ql,kl,D,causal,window,off,checks", FWD_CASES)
def test_page_forward_case(sec, B, H, Hkv, ql, kl, D, causal, window, off, checks):
    print(f"case page section {sec}", flush=True)
    q = fagen.lcg_bf16(SEED + off, (B, H, ql, D))
    k = fagen.lcg_bf16(SEED + off + 1, (B, Hkv, kl, D))
    v = fagen.lcg_bf16(SEED + off + 2, (B, Hkv, kl, D))
    mask = None if window is None else _swa_mask_bf16(B, H, ql, kl, window)
    o, l, bits = _forward(q, k, v, mask, B, H, Hkv, ql, kl, D, causal)
    of, ob, lr = oracle.fwd(q, k, v, None if mask is None else gu.widen(mask), B, H, Hkv, ql, kl,
                           D, 1.0 / math.sqrt(D), causal)
    eo = float(np.abs(o - gu.widen(ob)).max())
    el = float(np.abs(l - lr).max())
    print(f"page section {sec}: max|dO|={eo:.3e} max|dL|={el:.3e}")
    assert not np.isnan(o).any() and not np.isnan(l).any()
    if "O" in checks:
        assert eo <= 5e-3, eo
    if "L" in checks:
        assert el <= 3e-3, el


def test_page_forward_causal_sentinel():
    """Section 6: key rows after query 15 set to 128.0 must not change
    output rows 0..15 under causal masking (GPU on the perturbed keys
    against the oracle on the clean ones, 5e-3)."""
    B, H, Hkv, ql, kl, D, target = 1, 1, 1, 32, 32, 64, 15
    print("case page section 6 causal sentinel", flush=True)
    q = fagen.lcg_bf16(SEED + 40, (B, H, ql, D))
    k_f32 = fagen.lcg_f32(SEED + 41, (B, Hkv, kl, D))
    v = fagen.lcg_bf16(SEED + 42, (B, Hkv, kl, D))
    k_pert = k_f32.copy()
    k_pert[:, :, target + 1:, :] = 128.0
    k_clean_bits, k_pert_bits = _round(k_f32), _round(k_pert)
    o, _, _ = _forward(q, k_pert_bits, v, None, B, H, Hkv, ql, kl, D, True)
    _, ob, _ = oracle.fwd(q, k_clean_bits, v, None, B, H, Hkv, ql, kl, D, 1.0 / math.sqrt(D),
                          True)
    err = float(np.abs(o[:, :, :target + 1] - gu.widen(ob)[:, :, :target + 1]).max())
    print(f"page section 6: rows 0..{target} max|dO|={err:.3e}")
    assert err <= 5e-3


def _round(x):
    """f32 -> bf16 bits (round to nearest even), through torch."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


BWD_CASES = [
    # (section, B, H, Hkv, ql, kl, D, causal, window, seed offset)
    ("11 backward D=64", 1, 1, 1, 32, 32, 64, False, None, 100),
    ("12 backward D=256", 1, 4, 4, 128, 128, 256, False, None, 110),
    ("14 backward causal", 1, 1, 1, 64, 64, 64, True, None, 300),
    ("15 backward sliding window mask", 1, 1, 1, 32, 32, 64, False, 8, 400),
    ("16 backward GQA", 1, 8, 2, 32, 32, 64, False, None, 500),
]


@pytest.mark.parametrize("sec,B,H,Hkv,ql,kl,D,causal,window,off", BWD_CASES)
def test_page_backward_case(sec, B, H, Hkv, ql, kl, D, causal, window, off):
    import torch
    print(f"case page section {sec}", flush=True)
    scale = 1.0 / math.sqrt(D)
    q = fagen.lcg_bf16(SEED + off, (B, H, ql, D))
    k = fagen.lcg_bf16(SEED + off + 1, (B, Hkv, kl, D))
    v = fagen.lcg_bf16(SEED + off + 2, (B, Hkv, kl, D))
    g = fagen.lcg_bf16(SEED + off + 3, (B, H, ql, D))
    mask_bits = None if window is None else _swa_mask_bf16(B, H, ql, kl, window)
    qd, kd, vd, gd = _dev(q), _dev(k), _dev(v), _dev(g)
    md = None if mask_bits is None else _dev(mask_bits)
    # the page's chain: the GPU forward, then the GPU backward on its O and L
    O, L = fa.train_fwd_ex(qd, kd, vd, mask=md, scale=scale, causal=causal)
    dQ, dK, dV = fa.train_bwd_ex(qd, kd, vd, O, L, gd, mask=md, scale=scale, causal=causal)
    torch.cuda.synchronize()
    mask_f = None if mask_bits is None else gu.widen(mask_bits)
    _, _, lr = oracle.fwd(q, k, v, mask_f, B, H, Hkv, ql, kl, D, scale, causal)
    ref = oracle.bwd(q, k, v, mask_f, lr, g, B, H, Hkv, ql, kl, D, scale, causal)
    errs = []
    for name, got, r in zip(("dQ", "dK", "dV"), (dQ, dK, dV), ref):
        e = float(np.abs(got.float().cpu().numpy() - r).max())
        errs.append(e)
        print(f"page section {sec}: {name} max err {e:.3e} (max |ref| {np.abs(r).max():.3e})")
    assert max(errs) <= 5e-3, errs


def test_page_backward_finite_difference():
    """Section 13: d(sum O * dO)/dx at Q[0], K[0], V[0] from central
    differences (step 1e-2) of the oracle's forward on the f32 inputs,
    against the GPU's dQ, dK, dV there, within 5e-2."""
    import torch
    print("case page section 13 finite differences", flush=True)
    B, H, Hkv, ql, kl, D = 1, 1, 1, 8, 8, 64
    scale, h = 1.0 / math.sqrt(D), 1e-2
    qf = fagen.lcg_f32(SEED + 200, (B, H, ql, D))
    kf = fagen.lcg_f32(SEED + 201, (B, Hkv, kl, D))
    vf = fagen.lcg_f32(SEED + 202, (B, Hkv, kl, D))
    gf = fagen.lcg_f32(SEED + 203, (B, H, ql, D))
    qd, kd, vd, gd = (_dev(_round(x)) for x in (qf, kf, vf, gf))
    O, L = fa.train_fwd(qd, kd, vd, scale=scale)
    dQ, dK, dV = fa.train_bwd(qd, kd, vd, O, L, gd, scale=scale)
    torch.cuda.synchronize()

    def loss(q_, k_, v_):
        o = oracle.fwd(q_, k_, v_, None, B, H, Hkv, ql, kl, D, scale, False)[0]
        return float((o.astype(np.float32) * gf).sum(dtype=np.float32))

    for name, base, grad in (("dQ", qf, dQ), ("dK", kf, dK), ("dV", vf, dV)):
        plus, minus = base.copy(), base.copy()
        plus.reshape(-1)[0] += np.float32(h)
        minus.reshape(-1)[0] -= np.float32(h)
        args_p = {"dQ": (plus, kf, vf), "dK": (qf, plus, vf), "dV": (qf, kf, plus)}[name]
        args_m = {"dQ": (minus, kf, vf), "dK": (qf, minus, vf), "dV": (qf, kf, minus)}[name]
        fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
        an = float(grad.float().cpu().numpy().reshape(-1)[0])
        print(f"page section 13: {name}[0] finite difference {fd:.5f}, GPU {an:.5f}")
        assert abs(fd - an) <= 5e-2
