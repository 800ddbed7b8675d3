"""Invariants of the HIP forward that hold bit for bit on the GPU (no atomics,
no cross-workgroup communication, a fixed reduction order per row)."""
import numpy as np
import pytest

import fagen
import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _dev(a):
    return gu.to_dev(a, "cuda:0")


def _fwd(q, k, v, mask=None, scale=0.125, causal=True):
    import torch
    import flash_attention_forward_fa_amd as fa
    O, L = fa.train_fwd(q, k, v, mask=mask, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return O.view(torch.int16).cpu().numpy().view(np.uint16), L.cpu().numpy()


@pytest.mark.parametrize("D", [64, 128, 256])
def test_causal_sentinel_falsifier(D):
    """The method page's section 6 check, at GPU tile sizes: K rows after a
    target query set to 128.0 leave O rows 0..target bit-identical."""
    print(f"case sentinel D={D}", flush=True)
    B, H, ql, kl = 1, 2, 300, 300
    q = fagen.normal_bf16(11, 0, (B, H, ql, D))
    k = fagen.normal_bf16(11, 1, (B, H, kl, D))
    v = fagen.normal_bf16(11, 2, (B, H, kl, D))
    for target in (15, 63, 64, 200):
        kp = k.copy()
        kp[:, :, target + 1:] = 0x4300  # 128.0 in bf16
        a = _fwd(_dev(q), _dev(k), _dev(v), scale=D ** -0.5)
        b = _fwd(_dev(q), _dev(kp), _dev(v), scale=D ** -0.5)
        assert np.array_equal(a[0][:, :, :target + 1], b[0][:, :, :target + 1]), target
        assert np.array_equal(a[1][:, :, :target + 1], b[1][:, :, :target + 1]), target


@pytest.mark.parametrize("ql,kl", [(200, 333), (1, 333), (1, 64), (1, 1000)])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_gqa_equals_repeated_mha(D, ql, kl):
    """Also for one query row per head (decoding), where the GQA call runs the
    group's query heads as the rows of one packed head and the repeated-MHA
    call does not: the same bits."""
    print(f"case gqa D={D} ql={ql} kl={kl}", flush=True)
    B, H, Hkv = 2, 8, 2
    q = fagen.normal_bf16(12, 0, (B, H, ql, D))
    k = fagen.normal_bf16(12, 1, (B, Hkv, kl, D))
    v = fagen.normal_bf16(12, 2, (B, Hkv, kl, D))
    g = H // Hkv
    a = _fwd(_dev(q), _dev(k), _dev(v))
    b = _fwd(_dev(q), _dev(np.repeat(k, g, 1)), _dev(np.repeat(v, g, 1)))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_batch_and_head_slices_and_repeat_runs_are_identical():
    print("case slicing", flush=True)
    D, B, H, ql, kl = 64, 3, 4, 257, 257
    q = fagen.normal_bf16(13, 0, (B, H, ql, D))
    k = fagen.normal_bf16(13, 1, (B, H, kl, D))
    v = fagen.normal_bf16(13, 2, (B, H, kl, D))
    full = _fwd(_dev(q), _dev(k), _dev(v))
    again = _fwd(_dev(q), _dev(k), _dev(v))
    assert np.array_equal(full[0], again[0]) and np.array_equal(full[1], again[1])
    for b in range(B):
        one = _fwd(_dev(q[b:b + 1].copy()), _dev(k[b:b + 1].copy()), _dev(v[b:b + 1].copy()))
        assert np.array_equal(one[0], full[0][b:b + 1]) and np.array_equal(one[1], full[1][b:b + 1])
    one = _fwd(_dev(q[:, 2:3].copy()), _dev(k[:, 2:3].copy()), _dev(v[:, 2:3].copy()))
    assert np.array_equal(one[0], full[0][:, 2:3])


def test_zero_mask_matches_no_mask():
    print("case zero mask", flush=True)
    w = fagen.Workload("zm", 1, 2, 2, 96, 200, 64, True, seed_offset=3000)
    inp = fagen.generate(w)
    o1, l1, b1 = gu.run(inp, w)
    inp2 = dict(inp, mask=np.zeros((w.B, w.H, w.ql, w.kl), np.float32))
    o2, l2, b2 = gu.run(inp2, w)
    assert np.abs(o1 - o2).max() <= 5e-3 and np.abs(l1 - l2).max() <= 3e-3


def test_dominant_key_gives_one_hot_rows():
    """A key whose score exceeds all others by ~290 in base 2 (beyond exp2's
    f32 range): O equals its V row bit for bit, L its natural-log score."""
    print("case dominant key", flush=True)
    D, ql, kl = 64, 70, 70
    q = np.zeros((1, 1, ql, D), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, kl, D), np.float32)
    k[0, 0, :, 0] = np.linspace(-1, 1, kl)
    k[0, 0, kl - 1, 0] = 100.0
    v = fagen.normal_bf16(14, 2, (1, 1, kl, D))
    qb = (q.view(np.uint32) >> 16).astype(np.uint16)
    kb = (k.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    o, l = _fwd(_dev(qb), _dev(kb), _dev(v), scale=2.0, causal=False)
    assert np.array_equal(o[0, 0], np.broadcast_to(v[0, 0, kl - 1], (ql, D)))
    s = 2.0 * 100.0
    assert np.abs(l[0, 0] - s).max() <= 1e-4
    of, ob, lr = oracle.fwd(qb, kb, v, None, 1, 1, 1, ql, kl, D, 2.0, False)
    assert np.array_equal(o, ob)
