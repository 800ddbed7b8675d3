"""GPU tests of fa_train_fwd_strided (marked gpu): Q, K, V and O as strided
views — the sequence-major layout [B, L, H, D] seen as [B, H, L, D] (the
transposed K/V views of the adjacent attention API on the pages), slices of a
packed QKV tensor, a strided output. Only the addressing differs from the
contiguous kernels, so O and L must equal theirs bit for bit (plain, causal,
windowed, split-KV, the packed GQA decode); one case is also checked against
the oracle directly.
"""
import math

import numpy as np
import pytest

import fagen
import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _bshd(x):
    """A contiguous [B, H, L, D] device tensor -> the same values as a
    [B, H, L, D] view of a [B, L, H, D] tensor."""
    return x.transpose(1, 2).contiguous().transpose(1, 2)


def _inputs(seed, B, H, Hkv, ql, kl, D):
    dev = "cuda:0"
    return (gu.to_dev(fagen.normal_bf16(seed, 0, (B, H, ql, D)), dev),
            gu.to_dev(fagen.normal_bf16(seed, 1, (B, Hkv, kl, D)), dev),
            gu.to_dev(fagen.normal_bf16(seed, 2, (B, Hkv, kl, D)), dev))


def _same(a, b):
    import torch
    (o1, l1), (o2, l2) = a, b
    assert torch.equal(o1.contiguous().view(torch.int16), o2.contiguous().view(torch.int16))
    assert torch.equal(l1, l2)


CASES = [
    # (B, H, Hkv, ql, kl, D, causal, window)
    (2, 4, 2, 300, 300, 64, True, None),
    (1, 8, 2, 77, 513, 64, False, None),
    (2, 4, 4, 200, 260, 128, True, None),
    (1, 4, 1, 129, 129, 256, True, None),
    (2, 4, 2, 333, 333, 64, True, 100),
    (1, 2, 2, 300, 500, 256, True, 64),
    (3, 8, 2, 1, 700, 128, True, None),   # decoding: the packed GQA path
]


@pytest.mark.parametrize("B,H,Hkv,ql,kl,D,causal,window", CASES)
def test_bshd_views_equal_contiguous(B, H, Hkv, ql, kl, D, causal, window):
    import torch
    import flash_attention_forward_fa_amd as fa
    case = (B, H, Hkv, ql, kl, D, causal, window)
    print(f"case strided {case}", flush=True)
    q, k, v = _inputs(fagen.SEED_BASE + 14000 + CASES.index(case), B, H, Hkv, ql, kl, D)
    ref = fa.train_fwd_ex(q, k, v, causal=causal, window=window)
    qs, ks, vs = _bshd(q), _bshd(k), _bshd(v)
    # (a size-1 dimension keeps torch's own stride)
    assert (ql == 1 or qs.stride(2) == H * D) and ks.stride(2) == Hkv * D
    out = torch.empty(B, ql, H, D, dtype=torch.bfloat16, device="cuda:0").transpose(1, 2)
    got = fa.train_fwd_strided(qs, ks, vs, causal=causal, window=window, out=out)
    got2 = fa.train_fwd_strided(qs, ks, vs, causal=causal, window=window)  # contiguous O
    torch.cuda.synchronize()
    _same(ref, got)
    _same(ref, got2)
    if window is None:
        n = fa.suggest_n_split(B, H, ql, D, n_kv_heads=Hkv)
        if n > 1:
            refs = fa.train_fwd_split(q, k, v, n, causal=causal)
            gots = fa.train_fwd_strided(qs, ks, vs, causal=causal, n_split=n, out=out)
            torch.cuda.synchronize()
            _same(refs, gots)


def test_packed_qkv_slices_and_oracle():
    """Q, K, V as slices of one packed [B, L, 3, H, D] tensor (batch stride
    3*L*H*D, head stride D, row stride 3*H*D), against the contiguous kernel
    and the oracle."""
    import torch
    import flash_attention_forward_fa_amd as fa
    B, H, L, D = 2, 4, 200, 64
    print("case strided packed qkv", flush=True)
    seed = fagen.SEED_BASE + 14100
    qkv_np = fagen.normal_bf16(seed, 0, (B, L, 3, H, D))
    qkv = gu.to_dev(qkv_np, "cuda:0")
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    assert q.stride() == (3 * L * H * D, D, 3 * H * D, 1)
    got = fa.train_fwd_strided(q, k, v, causal=True)
    ref = fa.train_fwd(q.contiguous(), k.contiguous(), v.contiguous(), causal=True)
    torch.cuda.synchronize()
    _same(ref, got)
    qn, kn, vn = (np.ascontiguousarray(qkv_np[:, :, i].transpose(0, 2, 1, 3)) for i in range(3))
    of, ob, lr = oracle.fwd(qn, kn, vn, None, B, H, H, L, L, D, 1.0 / math.sqrt(D), True)
    o, l = got
    bits = o.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    eo, el, _ = gu.compare(gu.widen(bits), l.cpu().numpy(), bits, ob, lr, 5e-3, 3e-3,
                           "strided packed qkv", o_ref_f32=of)
    print(f"strided packed qkv: dO={eo:.3e} dL={el:.3e}")


def test_strided_errors_raise_from_binding():
    import torch
    import flash_attention_forward_fa_amd as fa
    q = torch.zeros(1, 2, 4, 64, device="cuda:0", dtype=torch.bfloat16)
    with pytest.raises(fa.FAError) as e:
        fa.train_fwd_strided(q, q, q, causal=False, window=3)
    assert e.value.status == 9
    odd = torch.zeros(1, 4, 2, 68, device="cuda:0", dtype=torch.bfloat16)[..., :64]
    with pytest.raises(fa.FAError) as e:   # row stride 68: not 16-byte rows
        fa.train_fwd_strided(odd.transpose(1, 2), q, q)
    assert e.value.status == 6


BWD_CASES = [
    # (B, H, Hkv, ql, kl, D, causal, window)
    (2, 4, 2, 300, 300, 64, True, None),
    (1, 4, 4, 77, 200, 64, False, None),
    (2, 8, 2, 200, 260, 128, True, None),
    (1, 4, 1, 129, 129, 256, True, None),
    (1, 4, 2, 333, 333, 64, True, 100),
    (1, 2, 2, 150, 300, 256, True, 64),
]


@pytest.mark.parametrize("B,H,Hkv,ql,kl,D,causal,window", BWD_CASES)
def test_backward_on_bshd_views_equals_contiguous(B, H, Hkv, ql, kl, D, causal, window):
    """fa_train_bwd_strided on [B, L, H, D] views of Q, K, V, O, dO gives the
    contiguous backward's dQ, dK, dV bits (written in the views' layout)."""
    import torch
    import flash_attention_forward_fa_amd as fa
    case = (B, H, Hkv, ql, kl, D, causal, window)
    print(f"case strided bwd {case}", flush=True)
    seed = fagen.SEED_BASE + 14200 + BWD_CASES.index(case)
    q, k, v = _inputs(seed, B, H, Hkv, ql, kl, D)
    dO = gu.to_dev(fagen.normal_bf16(seed, 6, (B, H, ql, D)), "cuda:0")
    O, L = fa.train_fwd_ex(q, k, v, causal=causal, window=window)
    ref = fa.train_bwd_ex(q, k, v, O, L, dO, causal=causal, window=window)
    qs, ks, vs, Os, dOs = (_bshd(x) for x in (q, k, v, O, dO))
    got = fa.train_bwd_strided(qs, ks, vs, Os, L, dOs, causal=causal, window=window)
    torch.cuda.synchronize()
    assert got[0].stride() == qs.stride() and got[1].stride() == ks.stride()
    for x, y in zip(ref, got):
        assert torch.equal(x.view(torch.int16), y.contiguous().view(torch.int16))


@pytest.mark.parametrize("kind", ["f32", "bf16", "bool"])
def test_sliced_mask_equals_contiguous(kind):
    """A mask sliced from a larger buffer ([1, H, 512, 512][..., :ql, :kl]: row
    stride 512) with Q, K, V, O, dO as [B, L, H, D] views: forward and backward
    bit-identical to fa_train_fwd_ex / fa_train_bwd_ex given the same mask made
    contiguous."""
    import torch
    import flash_attention_forward_fa_amd as fa
    from tests.pins import _finite_mask
    B, H, Hkv, ql, kl, D = 2, 4, 2, 200, 300, 64
    print(f"case strided sliced mask {kind}", flush=True)
    seed = fagen.SEED_BASE + 14300
    q, k, v = _inputs(seed, B, H, Hkv, ql, kl, D)
    dO = gu.to_dev(fagen.normal_bf16(seed, 6, (B, H, ql, D)), "cuda:0")
    big = _finite_mask(seed, 1, H, 512, 512)
    if kind == "bool":
        big_t = torch.from_numpy(np.isfinite(big)).cuda()
    elif kind == "bf16":
        bits = (np.ascontiguousarray(big).view(np.uint32) >> 16).astype(np.uint16)
        big_t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        big_t = torch.from_numpy(big).cuda()
    m = big_t[:, :, :ql, :kl]
    assert m.stride(2) == 512
    mc = m.contiguous()
    O1, L1 = fa.train_fwd_ex(q, k, v, mask=mc, causal=True)
    g1 = fa.train_bwd_ex(q, k, v, O1, L1, dO, mask=mc, causal=True)
    qs, ks, vs, dOs = (_bshd(x) for x in (q, k, v, dO))
    O2, L2 = fa.train_fwd_strided(qs, ks, vs, mask=m, causal=True,
                                  out=_bshd(torch.empty_like(q)))
    g2 = fa.train_bwd_strided(qs, ks, vs, O2, L2, dOs, mask=m, causal=True)
    torch.cuda.synchronize()
    _same((O1, L1), (O2, L2))
    for x, y in zip(g1, g2):
        assert torch.equal(x.view(torch.int16), y.contiguous().view(torch.int16))
