"""GPU parity of fa_train_fwd_ex's mask options against the CPU oracle (marked gpu):
bf16 masks (the dtype of the method page's harness), masks broadcast over
batch and/or heads (the [1, H, ql, kl] mask of the adjacent attention API on
the pages), strided masks, and their combination with causal and sliding-window
masking. The oracle always gets the equivalent dense f32 mask: a bf16 mask
widened exactly, a broadcast mask expanded.

The finite mask values here are N(0, 2^2) (natural-log units), far larger
than the workloads' 0/-inf masks: they concentrate the softmax, |O| reaches
|V|, and where O's exact value lies near a bf16 rounding boundary f32
evaluation order alone can move the rounded GPU and oracle outputs one bf16
step apart (2^-7 at |O| in [1, 2), more than 5e-3). An element may therefore
differ by one step; every other bound is the contract's.
"""
import numpy as np
import pytest

import fagen
import oracle
from tests import gpu_util as gu
from tests.pins import _finite_mask

pytestmark = pytest.mark.gpu


def _bf16_of(mask_f32):
    """bf16 bits of a mask whose values are bf16 numbers (or -inf): exact."""
    u = np.ascontiguousarray(mask_f32, np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


def _dev_mask(mask_f32, bf16):
    import torch
    if bf16:
        return torch.from_numpy(_bf16_of(mask_f32).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(mask_f32)).cuda()


def _run_ex(inp, w, mask_dev, causal, window=None):
    import torch
    import flash_attention_forward_fa_amd as fa
    q, k, v = (gu.to_dev(inp[n], "cuda:0") for n in ("q", "k", "v"))
    O, L = fa.train_fwd_ex(q, k, v, mask=mask_dev, scale=w.scale, causal=causal, window=window)
    torch.cuda.synchronize()
    bits = O.view(torch.int16).cpu().numpy().view(np.uint16)
    return gu.widen(bits), L.cpu().numpy(), bits


CASES = [
    # (B, H, Hkv, ql, kl, D, causal, window, mask batch, mask heads)
    (2, 4, 4, 64, 256, 64, True, None, 2, 4),    # the masked workload's shape
    (2, 4, 2, 100, 130, 64, False, None, 1, 4),  # one mask for every batch
    (3, 2, 1, 77, 77, 64, True, None, 1, 1),     # one mask for every batch and head
    (2, 2, 2, 90, 200, 64, True, 50, 1, 2),      # with a sliding window
    (2, 4, 1, 64, 96, 256, True, None, 2, 4),
    (2, 2, 2, 130, 130, 256, False, None, 1, 1),
    (1, 2, 1, 70, 300, 256, True, 100, 1, 2),
    (2, 2, 1, 80, 160, 128, True, None, 1, 2),
]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("B,H,Hkv,ql,kl,D,causal,window,mb,mh", CASES)
def test_mask_options_match_oracle(B, H, Hkv, ql, kl, D, causal, window, mb, mh, bf16):
    w = fagen.Workload("mask_ex", B, H, Hkv, ql, kl, D, causal,
                       seed_offset=6000 + ql + kl + D + mb * 10 + mh)
    print(f"case mask {(B, H, Hkv, ql, kl, D, causal, window, mb, mh)} bf16={bf16}", flush=True)
    inp = fagen.generate(w)
    m = _finite_mask(w.seed, mb, mh, ql, kl)
    dense = np.broadcast_to(m, (B, H, ql, kl)).copy()
    o, l, bits = _run_ex(inp, w, _dev_mask(m, bf16), causal, window)
    of, ob, lr = oracle.fwd(inp["q"], inp["k"], inp["v"], dense, B, H, Hkv, ql, kl, D, w.scale,
                            causal, window=window)
    tol_o, tol_l = gu.tolerances(kl)
    eo, el, rms = gu.compare(o, l, bits, ob, lr, tol_o, tol_l, f"mask {B,H,ql,kl,D} bf16={bf16}",
                             o_ref_f32=of)
    assert rms <= 2e-3, rms
    print(f"mask {(B, H, ql, kl, D, mb, mh)} bf16={bf16}: dO={eo:.3e} dL={el:.3e} "
          f"empty rows={int(np.isneginf(lr).sum())}")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_bf16_and_f32_masks_of_equal_values_give_equal_bits(D):
    """A 0/-inf mask has the same values in bf16 and f32: the two kernels
    compute the same numbers, so O and L agree bit for bit; the plain
    fa_train_fwd with the f32 mask does too."""
    import torch
    import flash_attention_forward_fa_amd as fa
    w = fagen.Workload("mask_eq", 2, 4, 4, 64, 256, D, True, mask_p=0.1, mask_full_rows=4,
                       seed_offset=6100 + D)
    print(f"case mask bits D={D}", flush=True)
    inp = fagen.generate(w)
    q, k, v = (gu.to_dev(inp[n], "cuda:0") for n in ("q", "k", "v"))
    o1, l1 = fa.train_fwd(q, k, v, mask=_dev_mask(inp["mask"], False), scale=w.scale, causal=True)
    o2, l2 = fa.train_fwd_ex(q, k, v, mask=_dev_mask(inp["mask"], False), scale=w.scale,
                             causal=True)
    o3, l3 = fa.train_fwd_ex(q, k, v, mask=_dev_mask(inp["mask"], True), scale=w.scale,
                             causal=True)
    torch.cuda.synchronize()
    for o, l in ((o2, l2), (o3, l3)):
        assert torch.equal(o1.view(torch.int16), o.view(torch.int16))
        assert torch.equal(l1, l)


def test_expanded_and_strided_masks():
    """A mask given as an expanded view (batch and head strides 0) and as a
    slice of a larger tensor (batch stride larger than H*ql*kl) reads the
    right elements: bit-identical to the same mask made dense."""
    import torch
    import flash_attention_forward_fa_amd as fa
    B, H, ql, kl, D = 2, 3, 70, 150, 64
    w = fagen.Workload("mask_view", B, H, 1, ql, kl, D, True, seed_offset=6200)
    print("case mask views", flush=True)
    inp = fagen.generate(w)
    q, k, v = (gu.to_dev(inp[n], "cuda:0") for n in ("q", "k", "v"))
    one = _dev_mask(_finite_mask(w.seed, 1, 1, ql, kl), True)
    dense = one.expand(B, H, ql, kl).contiguous()
    ref = fa.train_fwd_ex(q, k, v, mask=dense, scale=w.scale, causal=True)
    got = fa.train_fwd_ex(q, k, v, mask=one.expand(B, H, ql, kl), scale=w.scale, causal=True)
    big = _dev_mask(_finite_mask(w.seed + 1, B, 2 * H, ql, kl), False)
    sl = big[:, 1:H + 1]
    ref2 = fa.train_fwd_ex(q, k, v, mask=sl.contiguous(), scale=w.scale, causal=True)
    got2 = fa.train_fwd_ex(q, k, v, mask=sl, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    for (o1, l1), (o2, l2) in ((ref, got), (ref2, got2)):
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)


def test_ex_matches_the_other_entry_points_bit_for_bit():
    """fa_train_fwd_ex without a mask is fa_train_fwd (causal or not) and,
    with a window, fa_train_fwd_swa."""
    import torch
    import flash_attention_forward_fa_amd as fa
    w = fagen.Workload("ex_eq", 1, 4, 2, 300, 300, 64, True, seed_offset=6300)
    print("case ex equals", flush=True)
    inp = fagen.generate(w)
    q, k, v = (gu.to_dev(inp[n], "cuda:0") for n in ("q", "k", "v"))
    pairs = [(fa.train_fwd(q, k, v, causal=c), fa.train_fwd_ex(q, k, v, causal=c))
             for c in (False, True)]
    pairs.append((fa.train_fwd_swa(q, k, v, 90), fa.train_fwd_ex(q, k, v, causal=True, window=90)))
    torch.cuda.synchronize()
    for (o1, l1), (o2, l2) in pairs:
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)


def test_broadcast_bf16_mask_at_scale_sampled_rows():
    """One bf16 [1, 1, ql, kl] mask shared by every batch and head of a 2k
    causal problem, against the oracle on sampled rows."""
    B, H, ql, kl, D = 2, 4, 2048, 2048, 64
    w = fagen.Workload("mask_big", B, H, H, ql, kl, D, True, seed_offset=6400)
    print("case mask 2k broadcast", flush=True)
    inp = fagen.generate(w)
    m = _finite_mask(w.seed, 1, 1, ql, kl)
    o, l, bits = _run_ex(inp, w, _dev_mask(m, True), True)
    rng = np.random.default_rng(6400)
    rows = np.unique(np.concatenate([np.arange(200), rng.integers(0, B * H * ql, 200),
                                     (B * H - 1) * ql + np.arange(ql - 64, ql)])).astype(np.int64)
    dense = np.broadcast_to(m, (B, H, ql, kl))
    of, ob, lr = oracle.fwd_rows(inp["q"], inp["k"], inp["v"], np.ascontiguousarray(dense), B,
                                 H, H, ql, kl, D, w.scale, True, rows)
    o2, l2, b2 = o.reshape(-1, D)[rows], l.reshape(-1)[rows], bits.reshape(-1, D)[rows]
    eo, el, rms = gu.compare(o2, l2, b2, ob, lr, 1e-2, 1e-2, "mask 2k broadcast", o_ref_f32=of)
    assert rms <= 2e-3, rms
    print(f"mask 2k broadcast: {rows.size} rows dO={eo:.3e} dL={el:.3e} relRMS={rms:.2e}")


def test_ex_errors_raise_from_binding():
    import torch
    import flash_attention_forward_fa_amd as fa
    q = torch.zeros(1, 2, 4, 64, device="cuda:0", dtype=torch.bfloat16)
    with pytest.raises(fa.FAError) as e:
        fa.train_fwd_ex(q, q, q, causal=False, window=3)
    assert e.value.status == 9
    with pytest.raises(ValueError):
        fa.train_fwd_ex(q, q, q, mask=torch.zeros(1, 3, 4, 4, device="cuda:0"))
    with pytest.raises(ValueError):
        fa.train_fwd_ex(q, q, q, mask=torch.zeros(1, 2, 4, 4, device="cuda:0", dtype=torch.half))


BOOL_CASES = [
    # (B, H, Hkv, ql, kl, D, causal, mask batch, mask heads)
    (2, 4, 4, 33, 45, 64, False, 1, 1),     # the adjacent API's [ql, kl] boolean mask shape
    (2, 4, 2, 100, 100, 128, True, 1, 1),
    (1, 2, 1, 64, 96, 256, True, 1, 2),
    (2, 2, 2, 70, 300, 64, False, 2, 2),    # dense boolean mask
]


@pytest.mark.parametrize("B,H,Hkv,ql,kl,D,causal,mb,mh", BOOL_CASES)
def test_boolean_mask_matches_oracle_and_the_additive_mask(B, H, Hkv, ql, kl, D, causal, mb, mh):
    """A boolean mask (True = visible) against the oracle with the equivalent
    0/-inf f32 mask, and bit for bit against the kernel given that f32 mask.
    Rows whose mask is all False are empty (O = +0, L = -inf)."""
    import torch
    import flash_attention_forward_fa_amd as fa
    w = fagen.Workload("mask_bool", B, H, Hkv, ql, kl, D, causal,
                       seed_offset=6500 + ql + kl + D + mb + mh)
    print(f"case bool mask {(B, H, Hkv, ql, kl, D, causal, mb, mh)}", flush=True)
    inp = fagen.generate(w)
    keep = np.isfinite(_finite_mask(w.seed, mb, mh, ql, kl, p=0.3))  # one all-False row per slice
    add = np.where(keep, 0.0, -np.inf).astype(np.float32)
    q, k, v = (gu.to_dev(inp[n], "cuda:0") for n in ("q", "k", "v"))
    Ob, Lb = fa.train_fwd_ex(q, k, v, mask=torch.from_numpy(keep).cuda(), scale=w.scale,
                             causal=causal)
    Of, Lf = fa.train_fwd_ex(q, k, v, mask=torch.from_numpy(add).cuda(), scale=w.scale,
                             causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(Ob.view(torch.int16), Of.view(torch.int16)) and torch.equal(Lb, Lf)
    bits = Ob.view(torch.int16).cpu().numpy().view(np.uint16)
    dense = np.broadcast_to(add, (B, H, ql, kl)).copy()
    of, ob, lr = oracle.fwd(inp["q"], inp["k"], inp["v"], dense, B, H, Hkv, ql, kl, D, w.scale,
                           causal)
    tol_o, tol_l = gu.tolerances(kl)
    eo, el, _ = gu.compare(gu.widen(bits), Lb.cpu().numpy(), bits, ob, lr, tol_o, tol_l,
                           f"bool mask {B,H,ql,kl,D}", o_ref_f32=of)
    assert np.isneginf(lr).any()
    print(f"bool mask {(B, H, ql, kl, D, causal, mb, mh)}: dO={eo:.3e} dL={el:.3e}")
