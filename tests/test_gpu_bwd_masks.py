"""GPU parity of fa_train_bwd_ex's mask options (marked gpu): bf16 and boolean
masks, masks broadcast over batch and/or heads, alone and with causal and
sliding-window masking. The forward runs through fa_train_fwd_ex with the same
mask, as a training step would; the backward oracle gets the equivalent dense
f32 mask (a bf16 mask widened exactly, a boolean mask as 0/-inf, a broadcast
mask expanded) and the oracle forward's L. Bounds as for the plain backward:
1e-2 times the largest reference gradient of the tensor (at least 1) per
element, relative RMS at most 4e-3 per tensor.
"""
import math

import numpy as np
import pytest

import fagen
import oracle
from tests import gpu_util as gu
from tests.pins import _finite_mask

pytestmark = pytest.mark.gpu


def _bf16_of(mask_f32):
    u = np.ascontiguousarray(mask_f32, np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


def _device_mask(m, kind):
    """m: f32 mask [mb, mh, ql, kl] -> the device tensor of the given kind."""
    import torch
    if kind == "bf16":
        return torch.from_numpy(_bf16_of(m).view(np.int16)).view(torch.bfloat16).cuda()
    if kind == "bool":
        return torch.from_numpy(np.isfinite(m)).cuda()
    return torch.from_numpy(np.ascontiguousarray(m)).cuda()


def _inputs(seed, B, H, Hkv, ql, kl, D):
    return (fagen.normal_bf16(seed, 0, (B, H, ql, D)), fagen.normal_bf16(seed, 1, (B, Hkv, kl, D)),
            fagen.normal_bf16(seed, 2, (B, Hkv, kl, D)), fagen.normal_bf16(seed, 6, (B, H, ql, D)))


def _fwd_bwd(q, k, v, dO, mask, scale, causal, window):
    import torch
    import flash_attention_forward_fa_amd as fa
    qd, kd, vd, gd = (gu.to_dev(x, "cuda:0") for x in (q, k, v, dO))
    O, L = fa.train_fwd_ex(qd, kd, vd, mask=mask, scale=scale, causal=causal, window=window)
    grads = fa.train_bwd_ex(qd, kd, vd, O, L, gd, mask=mask, scale=scale, causal=causal,
                            window=window)
    torch.cuda.synchronize()
    return grads


CASES = [
    # (B, H, Hkv, ql, kl, D, causal, window, mask batch, mask heads, kind)
    (2, 4, 4, 64, 256, 64, True, None, 2, 4, "bf16"),
    (2, 4, 2, 100, 130, 64, False, None, 1, 4, "bf16"),
    (3, 2, 1, 77, 77, 64, True, None, 1, 1, "bool"),
    (2, 2, 2, 90, 200, 64, True, 50, 1, 2, "bf16"),
    (2, 4, 1, 64, 96, 256, True, None, 2, 4, "bf16"),
    (2, 2, 2, 130, 130, 256, False, None, 1, 1, "bool"),
    (1, 2, 1, 70, 300, 256, True, 100, 1, 2, "bool"),
    (2, 2, 1, 80, 160, 128, True, None, 1, 2, "bf16"),
    (1, 4, 2, 150, 150, 128, False, None, 1, 1, "bool"),
    (2, 2, 2, 96, 96, 64, True, 30, 2, 1, "f32"),
]


@pytest.mark.parametrize("B,H,Hkv,ql,kl,D,causal,window,mb,mh,kind", CASES)
def test_backward_mask_options_match_oracle(B, H, Hkv, ql, kl, D, causal, window, mb, mh, kind):
    case = (B, H, Hkv, ql, kl, D, causal, window, mb, mh, kind)
    print(f"case bwd mask {case}", flush=True)
    seed = fagen.SEED_BASE + 12000 + CASES.index(case)
    q, k, v, dO = _inputs(seed, B, H, Hkv, ql, kl, D)
    m = _finite_mask(seed, mb, mh, ql, kl)
    if kind == "bool":
        m = np.where(np.isfinite(m), 0.0, -np.inf).astype(np.float32)
    dense = np.broadcast_to(m, (B, H, ql, kl)).copy()
    scale = 1.0 / math.sqrt(D)
    import torch
    got = [gu.widen(t.view(torch.int16).cpu().numpy().view(np.uint16))
           for t in _fwd_bwd(q, k, v, dO, _device_mask(m, kind), scale, causal, window)]
    _, _, Lr = oracle.fwd(q, k, v, dense, B, H, Hkv, ql, kl, D, scale, causal, window=window)
    ref = oracle.bwd(q, k, v, dense, Lr, dO, B, H, Hkv, ql, kl, D, scale, causal, window=window)
    for tname, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert not np.isnan(g).any(), f"NaN in {tname}"
        err = float(np.abs(g - r).max())
        bound = 1e-2 * max(1.0, float(np.abs(r).max()))
        rms = float(np.sqrt(np.mean((g - r) ** 2)) / max(np.sqrt(np.mean(r ** 2)), 1e-2))
        print(f"bwd mask {case}: {tname} {err:.2e}/{bound:.2e} rms {rms:.1e}", flush=True)
        assert err <= bound, f"{tname} max error {err:.3e} > {bound:.3e}"
        assert rms <= 4e-3, f"{tname} relative RMS error {rms:.2e}"


@pytest.mark.parametrize("D", [64, 128, 256])
def test_backward_mask_kinds_of_equal_values_give_equal_bits(D):
    """A 0/-inf mask given as f32 (fa_train_bwd), f32, bf16 and boolean
    (fa_train_bwd_ex), and as an expanded broadcast view, yields the same
    dQ, dK and dV bits."""
    import torch
    import flash_attention_forward_fa_amd as fa
    B, H, Hkv, ql, kl = 2, 4, 2, 96, 200
    print(f"case bwd mask bits D={D}", flush=True)
    seed = fagen.SEED_BASE + 12100 + D
    q, k, v, dO = (gu.to_dev(x, "cuda:0") for x in _inputs(seed, B, H, Hkv, ql, kl, D))
    m1, _ = fagen.mask_f32(seed, 1, H, ql, kl, 0.15, 2)
    one = torch.from_numpy(m1).cuda()
    dense = one.expand(B, H, ql, kl).contiguous()
    scale = 1.0 / math.sqrt(D)
    O, L = fa.train_fwd(q, k, v, mask=dense, scale=scale, causal=True)
    ref = fa.train_bwd(q, k, v, O, L, dO, mask=dense, scale=scale, causal=True)
    variants = [dense, one.expand(B, H, ql, kl), one.to(torch.bfloat16),
                torch.isfinite(one), torch.isfinite(dense)]
    outs = [fa.train_bwd_ex(q, k, v, O, L, dO, mask=mv, scale=scale, causal=True)
            for mv in variants]
    torch.cuda.synchronize()
    for i, got in enumerate(outs):
        for x, y in zip(ref, got):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16)), f"variant {i}"


def test_backward_ex_without_mask_matches_the_other_entry_points():
    """fa_train_bwd_ex without a mask is fa_train_bwd and, with a window,
    fa_train_bwd_swa, bit for bit."""
    import torch
    import flash_attention_forward_fa_amd as fa
    B, H, Hkv, ql, kl, D = 1, 4, 2, 200, 260, 64
    print("case bwd ex equals", flush=True)
    seed = fagen.SEED_BASE + 12200
    q, k, v, dO = (gu.to_dev(x, "cuda:0") for x in _inputs(seed, B, H, Hkv, ql, kl, D))
    pairs = []
    for c in (False, True):
        O, L = fa.train_fwd(q, k, v, causal=c)
        pairs.append((fa.train_bwd(q, k, v, O, L, dO, causal=c),
                      fa.train_bwd_ex(q, k, v, O, L, dO, causal=c)))
    O, L = fa.train_fwd_swa(q, k, v, 70)
    pairs.append((fa.train_bwd_swa(q, k, v, O, L, dO, 70),
                  fa.train_bwd_ex(q, k, v, O, L, dO, causal=True, window=70)))
    torch.cuda.synchronize()
    for a, b in pairs:
        for x, y in zip(a, b):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_backward_ex_errors_raise_from_binding():
    import torch
    import flash_attention_forward_fa_amd as fa
    q = torch.zeros(1, 2, 4, 64, device="cuda:0", dtype=torch.bfloat16)
    L = torch.zeros(1, 2, 4, device="cuda:0")
    with pytest.raises(fa.FAError) as e:
        fa.train_bwd_ex(q, q, q, q, L, q, causal=False, window=3)
    assert e.value.status == 9
    with pytest.raises(ValueError):
        fa.train_bwd_ex(q, q, q, q, L, q, mask=torch.zeros(1, 3, 4, 4, device="cuda:0"))
