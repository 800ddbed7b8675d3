"""GPU tests of offsets beyond 32 bits (marked gpu): every element offset in
the kernels is 64-bit, which these check where it matters.

- K and V of 136 heads x 131072 keys x head_dim 128 (4.6 GB each): the last
  head starts above 2^32 bytes, head 70 above 2^31. The forward, the split-KV
  forward and the backward are compared with the oracle on the heads that hold
  generated data (0, 70, 135); the other heads are zero, so a head that read
  another head's keys would differ.
- Masks whose batch stride exceeds 2^31 elements (boolean) or 2^31 bytes
  (f32), given as strided views of one large buffer: forward and backward
  bit-identical to the same mask made dense.
"""
import math

import numpy as np
import pytest

import fagen
import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

HEADS = (0, 70, 135)


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def test_kv_heads_beyond_4gib():
    import torch
    import flash_attention_forward_fa_amd as fa
    H, ql, kl, D = 136, 16, 131072, 128
    print(f"case large K/V: H{H} ql{ql} kl{kl} D{D}", flush=True)
    seed = fagen.SEED_BASE + 13000
    dev = "cuda:0"
    q_np = fagen.normal_bf16(seed, 0, (1, H, ql, D))
    do_np = fagen.normal_bf16(seed, 6, (1, H, ql, D))
    k = torch.zeros(1, H, kl, D, dtype=torch.bfloat16, device=dev)
    v = torch.zeros(1, H, kl, D, dtype=torch.bfloat16, device=dev)
    assert k.numel() * 2 > 2 ** 32
    kv = {}
    for h in HEADS:
        kv[h] = (fagen.normal_bf16(seed + h, 1, (1, 1, kl, D)),
                 fagen.normal_bf16(seed + h, 2, (1, 1, kl, D)))
        k[:, h:h + 1] = gu.to_dev(kv[h][0], dev)
        v[:, h:h + 1] = gu.to_dev(kv[h][1], dev)
    q, dO = gu.to_dev(q_np, dev), gu.to_dev(do_np, dev)
    scale = 1.0 / math.sqrt(D)
    O, L = fa.train_fwd(q, k, v, scale=scale)
    Os, Ls = fa.train_fwd_split(q, k, v, 64, scale=scale)
    dQ, dK, dV = fa.train_bwd(q, k, v, O, L, dO, scale=scale)
    torch.cuda.synchronize()
    print("large K/V: kernels done", flush=True)
    ob, l = _bits(O), L.cpu().numpy()
    obs, ls = _bits(Os), Ls.cpu().numpy()
    for h in HEADS:
        qh, doh = q_np[:, h:h + 1].copy(), do_np[:, h:h + 1].copy()
        kh, vh = kv[h]
        rf, rb, rl = oracle.fwd(qh, kh, vh, None, 1, 1, 1, ql, kl, D, scale, False)
        for name, bits, lv in (("plain", ob, l), ("split", obs, ls)):
            eo, el, _ = gu.compare(gu.widen(bits[:, h:h + 1]), lv[:, h:h + 1], bits[:, h:h + 1],
                                   rb, rl, 1e-2, 1e-2, f"large K/V {name} head {h}", o_ref_f32=rf)
            print(f"large K/V {name} head {h}: dO={eo:.3e} dL={el:.3e}", flush=True)
        ref = oracle.bwd(qh, kh, vh, None, rl, doh, 1, 1, 1, ql, kl, D, scale, False)
        got = [gu.widen(_bits(t[:, h:h + 1])) for t in (dQ, dK, dV)]
        for tname, g, r in zip(("dQ", "dK", "dV"), got, ref):
            err = float(np.abs(g - r).max())
            bound = 1e-2 * max(1.0, float(np.abs(r).max()))
            print(f"large K/V head {h}: {tname} {err:.2e}/{bound:.2e}", flush=True)
            assert err <= bound, f"head {h} {tname}: {err:.3e} > {bound:.3e}"
    # a zero head: uniform weights over zero values
    assert np.all(gu.widen(ob[:, 1]) == 0) and np.all(gu.widen(ob[:, H - 2]) == 0)
    del k, v, dK, dV
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kind", ["bool", "f32"])
def test_mask_batch_stride_beyond_2g(kind):
    import torch
    import flash_attention_forward_fa_amd as fa
    B, H, Hkv, ql, kl, D = 2, 2, 1, 64, 256, 64
    print(f"case large mask stride {kind}", flush=True)
    seed = fagen.SEED_BASE + 13100
    dev = "cuda:0"
    q, k, v, dO = (gu.to_dev(fagen.normal_bf16(seed, st, shp), dev) for st, shp in
                   ((0, (B, H, ql, D)), (1, (B, Hkv, kl, D)), (2, (B, Hkv, kl, D)),
                    (6, (B, H, ql, D))))
    m, _ = fagen.mask_f32(seed, B, H, ql, kl, 0.2, 2)
    if kind == "bool":
        dense = torch.from_numpy(np.isfinite(m)).to(dev)
        sb = 2 ** 31 + 256                       # elements = bytes
    else:
        dense = torch.from_numpy(m).to(dev)
        sb = 2 ** 29 + 64                        # 2^31 + 256 bytes
    buf = torch.zeros(sb + H * ql * kl, dtype=dense.dtype, device=dev)
    view = torch.as_strided(buf, (B, H, ql, kl), (sb, ql * kl, kl, 1))
    view.copy_(dense)
    assert view.stride(0) * view.element_size() > 2 ** 31
    O1, L1 = fa.train_fwd_ex(q, k, v, mask=dense, causal=True)
    O2, L2 = fa.train_fwd_ex(q, k, v, mask=view, causal=True)
    g1 = fa.train_bwd_ex(q, k, v, O1, L1, dO, mask=dense, causal=True)
    g2 = fa.train_bwd_ex(q, k, v, O1, L1, dO, mask=view, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16)) and torch.equal(L1, L2)
    for x, y in zip(g1, g2):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert torch.isneginf(L1).any()  # the full -inf rows are there
    del buf, view
    torch.cuda.empty_cache()
