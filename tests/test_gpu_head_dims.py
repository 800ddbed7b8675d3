"""Head dims 80, 96 and 192 and value widths that differ from the key width.

The shapes are those of the adjacent SDPA page ("nuvec-core 0.3.0",
tests/fast.rs, attention_kernels_match_the_fallback): (B, Hq, Hkv, Lq, Lk, D,
Dv) with D in {64, 80, 96, 128, 192} and the pairs (96, 64) and (192, 128),
each with no mask, the causal rule, a boolean mask and an additive mask
([1, Hq, Lq, Lk], broadcast over the batch), at scale 0.3. Beyond them, every
new (D, Dv) pair runs on shapes of several query and key tiles with ragged
tails (full, causal, sliding window, boolean and f32 masks), on a long one
that takes the plain (bf16 P) tiles, and on strided K/V views of
[B, L, H, D]. The HIP path runs through the C ABI (fa_train_fwd_dv, or
fa_train_fwd for D == Dv); the oracle is fa_oracle_fwd_general with the value
width. Inputs are seeded N(0, 1) bf16 (fagen). Bounds: those of the other
forward tests (O 5e-3 and L 3e-3 up to 256 keys, 1e-2 beyond, with the bf16
step rule of gpu_util.compare), tighter than the page's 5e-2 for bf16.
"""
import math

import numpy as np
import pytest

import fagen
import oracle
import flash_attention_forward_fa_amd as fa
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

PAGE_SHAPES = [
    (2, 4, 4, 1, 37, 64, 64), (1, 8, 2, 4, 50, 128, 128), (1, 4, 4, 2, 33, 96, 64),
    (1, 2, 1, 1, 20, 192, 128), (1, 8, 1, 1, 1100, 128, 128), (1, 16, 2, 1, 9000, 128, 128),
    (2, 4, 2, 33, 45, 64, 64), (1, 2, 2, 100, 100, 80, 80), (1, 4, 4, 64, 96, 128, 128),
    (1, 2, 2, 40, 40, 96, 64),
]
MASKS = ["none", "causal", "bool", "additive"]
PAIRS = [(80, 80), (96, 96), (96, 64), (192, 192), (192, 128)]


def _inputs(seed, B, H, Hkv, ql, kl, D, Dv):
    q = fagen.normal_bf16(seed, fagen.STREAM_Q, (B, H, ql, D))
    k = fagen.normal_bf16(seed, fagen.STREAM_K, (B, Hkv, kl, D))
    v = fagen.normal_bf16(seed, fagen.STREAM_V, (B, Hkv, kl, Dv))
    return q, k, v


def _mask(kind, seed, H, ql, kl):
    """(mask for the HIP call [1, H, ql, kl] or None, oracle mask f32 or None)."""
    if kind in ("none", "causal", "window"):
        return None, None
    if kind == "bool":
        add, _ = fagen.mask_f32(seed, 1, H, ql, kl, p_masked=0.2,
                                n_full_rows=1 if ql >= 4 else 0)
        return add == 0.0, add
    if kind == "additive":
        m = fagen.bf16_bits_to_f32(fagen.normal_bf16(seed, fagen.STREAM_MASK, (1, H, ql, kl)))
        return m, m
    add, _ = fagen.mask_f32(seed, 1, H, ql, kl, p_masked=0.1, n_full_rows=1 if ql >= 4 else 0)
    return add, add


def _run(case, q, k, v, D, Dv, scale, causal=False, window=None, mask=None, views=False):
    """The HIP forward and the oracle; compares them and returns the GPU O bits."""
    import torch
    B, H, ql, _ = q.shape
    Hkv, kl = k.shape[1], k.shape[2]
    print(f"case {case}", flush=True)
    dev = "cuda:0"
    tq, tk, tv = gu.to_dev(q, dev), gu.to_dev(k, dev), gu.to_dev(v, dev)
    if views:
        # K and V (and Q) as transposed views of sequence-major [B, L, H, D]
        tq = tq.transpose(1, 2).contiguous().transpose(1, 2)
        tk = tk.transpose(1, 2).contiguous().transpose(1, 2)
        tv = tv.transpose(1, 2).contiguous().transpose(1, 2)
    tm = None
    if mask is not None:
        tm = torch.from_numpy(np.ascontiguousarray(mask[0])).to(dev)
    O, L = fa.train_fwd_dv(tq, tk, tv, mask=tm, scale=scale, causal=causal, window=window)
    torch.cuda.synchronize()
    bits = O.view(torch.int16).cpu().numpy().view(np.uint16)
    om = None
    if mask is not None:
        om = np.ascontiguousarray(np.broadcast_to(mask[1], (B, H, ql, kl)), dtype=np.float32)
    of, ob, lr = oracle.fwd_dv(q, k, v, om, B, H, Hkv, ql, kl, D, Dv, scale,
                               causal or window is not None, window=window)
    tol_o, tol_l = gu.tolerances(kl)
    gu.compare(gu.widen(bits), L.cpu().numpy(), bits, ob, lr, tol_o, tol_l, label=case,
               o_ref_f32=of)
    return bits


@pytest.mark.parametrize("kind", MASKS)
@pytest.mark.parametrize("shape", PAGE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_page_shapes(shape, kind):
    B, H, Hkv, ql, kl, D, Dv = shape
    seed = fagen.SEED_BASE + 0x100 + PAGE_SHAPES.index(shape)
    q, k, v = _inputs(seed, B, H, Hkv, ql, kl, D, Dv)
    mask = _mask(kind, seed, H, ql, kl)
    _run(f"page shape {shape} {kind}", q, k, v, D, Dv, 0.3, causal=kind == "causal",
         mask=mask if mask[0] is not None else None)


@pytest.mark.parametrize("kind", ["none", "causal", "window", "bool", "f32"])
@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0]}-{p[1]}")
def test_pairs_ragged_tiles(pair, kind):
    # several query tiles (256 or 128 rows each) and key tiles (64 keys), both
    # with ragged tails; causal offset 33; GQA groups of 2
    D, Dv = pair
    B, H, Hkv, ql, kl = 2, 4, 2, 300, 333
    seed = fagen.SEED_BASE + 0x200 + 7 * PAIRS.index(pair)
    q, k, v = _inputs(seed, B, H, Hkv, ql, kl, D, Dv)
    mask = _mask(kind, seed, H, ql, kl)
    _run(f"pair {pair} {kind}", q, k, v, D, Dv, 1.0 / math.sqrt(D),
         causal=kind in ("causal", "window"), window=70 if kind == "window" else None,
         mask=mask if mask[0] is not None else None)


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0]}-{p[1]}")
def test_pairs_long_plain_tiles(pair):
    # more than 256 keys: the plain tiles (bf16 P, pre-scaled Q), their
    # compensated short first tiles and the redo of rows with |O| >= 1
    D, Dv = pair
    B, H, Hkv, ql, kl = 1, 4, 1, 640, 1100
    seed = fagen.SEED_BASE + 0x300 + PAIRS.index(pair)
    q, k, v = _inputs(seed, B, H, Hkv, ql, kl, D, Dv)
    _run(f"pair {pair} long causal", q, k, v, D, Dv, 1.0 / math.sqrt(D), causal=True)


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0]}-{p[1]}")
def test_pairs_strided_views(pair):
    D, Dv = pair
    B, H, Hkv, ql, kl = 2, 4, 2, 130, 200
    seed = fagen.SEED_BASE + 0x400 + PAIRS.index(pair)
    q, k, v = _inputs(seed, B, H, Hkv, ql, kl, D, Dv)
    _run(f"pair {pair} strided views", q, k, v, D, Dv, 1.0 / math.sqrt(D), causal=True,
         views=True)


@pytest.mark.parametrize("D", [80, 96, 192])
def test_same_width_entry_points_agree(D):
    # with Dv == D the plain entry point runs the same kernels: same bits
    import torch
    B, H, Hkv, ql, kl = 1, 4, 2, 200, 300
    seed = fagen.SEED_BASE + 0x500 + D
    q, k, v = _inputs(seed, B, H, Hkv, ql, kl, D, D)
    print(f"case same-width entry points D={D}", flush=True)
    tq, tk, tv = (gu.to_dev(x, "cuda:0") for x in (q, k, v))
    O1, L1 = fa.train_fwd(tq, tk, tv, causal=True)
    O2, L2 = fa.train_fwd_dv(tq, tk, tv, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16))
    assert torch.equal(L1, L2)


def test_unsupported_pairs_raise():
    import torch
    q = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16, device="cuda:0")
    k = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16, device="cuda:0")
    v = torch.zeros((1, 2, 8, 128), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(fa.FAError):
        fa.train_fwd_dv(q, k, v)
    k80 = torch.zeros((1, 2, 64, 80), dtype=torch.bfloat16, device="cuda:0")
    q80 = torch.zeros((1, 2, 8, 80), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(fa.FAError):
        fa.train_fwd_split(q80, k80, k80, n_split=2)
