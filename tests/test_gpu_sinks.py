"""Attention sinks on the GPU (fa_train_fwd_dv with a sinks array) against the
oracle's fa_oracle_fwd_sinks (marked gpu).

The adjacent SDPA page ("nuvec-core 0.3.0", the attention API) takes an
optional f32 `sinks [Hq]` without defining it; the reading both sides follow
is one logit per query head that joins every row's softmax as one more term
with a zero value: L = log(exp(sink) + sum_j exp(s_j)), O = sum_j exp(s_j - L)
v_j, and a row with no visible key has O = 0 and L = sink.

Sinks are drawn as log(kl) + N(0, 2^2) (rounded through bf16, so exact in
f32): near the log of the rows' key mass, where a sink moves both O and L by a
visible amount and a sink read for the wrong head or row fails the bounds.
Inputs otherwise as in the head-dim tests: seeded N(0, 1) bf16 (fagen), the
page's shapes and masks, multi-tile shapes with ragged tails, the long plain
(bf16 P) tiles, and the packed decode of GQA (one query row per head, where a
kv head's query heads become the rows of one packed head). Bounds: those of
the other forward tests.
"""
import math

import numpy as np
import pytest

import fagen
import oracle
import flash_attention_forward_fa_amd as fa
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

STREAM_SINKS = 5


def _inputs(seed, B, H, Hkv, ql, kl, D, Dv):
    q = fagen.normal_bf16(seed, fagen.STREAM_Q, (B, H, ql, D))
    k = fagen.normal_bf16(seed, fagen.STREAM_K, (B, Hkv, kl, D))
    v = fagen.normal_bf16(seed, fagen.STREAM_V, (B, Hkv, kl, Dv))
    return q, k, v


def _sinks(seed, H, kl, shift=None):
    z = fagen.bf16_bits_to_f32(fagen.normal_bf16(seed, STREAM_SINKS, (H,), sigma=2.0))
    base = math.log(max(kl, 1)) if shift is None else shift
    return (np.float32(base) + z).astype(np.float32)


def _mask(kind, seed, H, ql, kl):
    """(mask for the HIP call [1, H, ql, kl] or None, oracle mask f32 or None)."""
    if kind == "bool":
        add, _ = fagen.mask_f32(seed, 1, H, ql, kl, p_masked=0.2,
                                n_full_rows=1 if ql >= 4 else 0)
        return add == 0.0, add
    if kind == "additive":
        m = fagen.bf16_bits_to_f32(fagen.normal_bf16(seed, fagen.STREAM_MASK, (1, H, ql, kl)))
        return m, m
    return None, None


def _run(case, q, k, v, sinks, scale, causal=False, window=None, mask=(None, None)):
    """The HIP forward with sinks and the oracle; compares them; returns
    (O bits, L, oracle L)."""
    import torch
    B, H, ql, D = q.shape
    Hkv, kl, Dv = k.shape[1], k.shape[2], v.shape[3]
    print(f"case {case}", flush=True)
    dev = "cuda:0"
    tq, tk, tv = gu.to_dev(q, dev), gu.to_dev(k, dev), gu.to_dev(v, dev)
    ts = torch.from_numpy(sinks).to(dev)
    tm = None if mask[0] is None else torch.from_numpy(np.ascontiguousarray(mask[0])).to(dev)
    O, L = fa.train_fwd_dv(tq, tk, tv, mask=tm, scale=scale, causal=causal, window=window,
                           sinks=ts)
    torch.cuda.synchronize()
    bits = O.view(torch.int16).cpu().numpy().view(np.uint16)
    lg = L.cpu().numpy()
    om = None
    if mask[1] is not None:
        om = np.ascontiguousarray(np.broadcast_to(mask[1], (B, H, ql, kl)), dtype=np.float32)
    of, ob, lr = oracle.fwd_dv(q, k, v, om, B, H, Hkv, ql, kl, D, Dv, scale,
                               causal or window is not None, window=window, sinks=sinks)
    tol_o, tol_l = gu.tolerances(kl)
    eo, el, rms = gu.compare(gu.widen(bits), lg, bits, ob, lr, tol_o, tol_l, label=case,
                             o_ref_f32=of)
    print(f"{case}: dO={eo:.3e} dL={el:.3e} relRMS={rms:.2e}")
    return bits, lg, lr


PAGE_SHAPES = [
    (2, 4, 4, 1, 37, 64, 64), (1, 8, 2, 4, 50, 128, 128), (1, 4, 4, 2, 33, 96, 64),
    (1, 2, 1, 1, 20, 192, 128), (1, 8, 1, 1, 1100, 128, 128), (2, 4, 2, 33, 45, 64, 64),
    (1, 2, 2, 100, 100, 80, 80), (1, 2, 2, 40, 40, 96, 64),
]


@pytest.mark.parametrize("kind", ["none", "causal", "bool", "additive"])
@pytest.mark.parametrize("shape", PAGE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_sinks_page_shapes(shape, kind):
    B, H, Hkv, ql, kl, D, Dv = shape
    seed = fagen.SEED_BASE + 0x900 + PAGE_SHAPES.index(shape)
    q, k, v = _inputs(seed, B, H, Hkv, ql, kl, D, Dv)
    _run(f"sinks page shape {shape} {kind}", q, k, v, _sinks(seed, H, kl), 0.3,
         causal=kind == "causal", mask=_mask(kind, seed, H, ql, kl))


@pytest.mark.parametrize("kind", ["causal", "window", "bool"])
@pytest.mark.parametrize("pair", [(64, 64), (128, 128), (256, 256), (192, 128)],
                         ids=lambda p: f"{p[0]}-{p[1]}")
def test_sinks_ragged_tiles(pair, kind):
    # several query and key tiles with ragged tails; GQA groups of 2; the
    # bool mask hides whole rows (O = 0, L = the sink there)
    D, Dv = pair
    B, H, Hkv, ql, kl = 2, 4, 2, 300, 333
    seed = fagen.SEED_BASE + 0xA00 + D + Dv
    q, k, v = _inputs(seed, B, H, Hkv, ql, kl, D, Dv)
    s = _sinks(seed, H, kl)
    bits, lg, lr = _run(f"sinks pair {pair} {kind}", q, k, v, s, 1.0 / math.sqrt(D),
                        causal=kind in ("causal", "window"),
                        window=70 if kind == "window" else None,
                        mask=_mask(kind, seed, H, ql, kl))
    if kind == "bool":
        # rows that see no key: exactly +0 and the head's sink
        add, _ = fagen.mask_f32(seed, 1, H, ql, kl, p_masked=0.2, n_full_rows=1)
        empty = np.broadcast_to(np.all(np.isneginf(add), axis=-1), (B, H, ql))
        assert empty.any()
        assert np.all(bits[empty] == 0)
        hs = np.broadcast_to(np.arange(H)[None, :, None], (B, H, ql))[empty]
        np.testing.assert_allclose(lg[empty], s[hs], rtol=0, atol=1e-5)


@pytest.mark.parametrize("pair", [(64, 64), (128, 128), (256, 256), (96, 64)],
                         ids=lambda p: f"{p[0]}-{p[1]}")
def test_sinks_long_plain_tiles(pair):
    # more than 256 keys: plain tiles, their compensated short first tiles and
    # the redo of rows with |O| >= 1, with the sink folded in at the end
    D, Dv = pair
    B, H, Hkv, ql, kl = 1, 4, 1, 640, 1100
    seed = fagen.SEED_BASE + 0xB00 + D + Dv
    q, k, v = _inputs(seed, B, H, Hkv, ql, kl, D, Dv)
    _run(f"sinks pair {pair} long causal", q, k, v, _sinks(seed, H, kl), 1.0 / math.sqrt(D),
         causal=True)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_sinks_packed_gqa_decode(D):
    # one query row per head on 8 kv heads of 4 query heads each: the query
    # heads are packed as rows, each row still takes its own head's sink
    B, H, Hkv, ql, kl = 2, 32, 8, 1, 5000
    seed = fagen.SEED_BASE + 0xC00 + D
    q, k, v = _inputs(seed, B, H, Hkv, ql, kl, D, D)
    s = _sinks(seed, H, kl)
    _, lg, lr = _run(f"sinks packed decode D={D}", q, k, v, s, 1.0 / math.sqrt(D), causal=True)
    # the sinks matter: without them L drops by log(1 + exp(sink - L_keys))
    of, ob, l0 = oracle.fwd_dv(q, k, v, None, B, H, Hkv, ql, kl, D, D, 1.0 / math.sqrt(D), True)
    assert np.abs(lg - l0).max() > 0.5


def test_sinks_dominant_minus_inf_and_no_keys():
    """A sink far above every score leaves O near 0 and L near the sink; -inf
    sinks give the bits of no sinks; with no keys at all O = +0, L = sink."""
    import torch
    B, H, Hkv, ql, kl, D = 1, 4, 2, 200, 700, 128
    seed = fagen.SEED_BASE + 0xD00
    q, k, v = _inputs(seed, B, H, Hkv, ql, kl, D, D)
    _run("sinks dominant", q, k, v, _sinks(seed, H, kl, shift=40.0), 1.0 / math.sqrt(D),
         causal=True)
    print("case sinks -inf", flush=True)
    tq, tk, tv = (gu.to_dev(x, "cuda:0") for x in (q, k, v))
    neg = torch.full((H,), -math.inf, dtype=torch.float32, device="cuda:0")
    O1, L1 = fa.train_fwd_dv(tq, tk, tv, causal=True)
    O2, L2 = fa.train_fwd_dv(tq, tk, tv, causal=True, sinks=neg)
    torch.cuda.synchronize()
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16))
    assert torch.equal(L1, L2)
    print("case sinks kl=0", flush=True)
    s = torch.from_numpy(_sinks(seed, H, 0)).to("cuda:0")
    k0 = torch.empty((B, Hkv, 0, D), dtype=torch.bfloat16, device="cuda:0")
    O3, L3 = fa.train_fwd_dv(tq, k0, k0, causal=True, sinks=s)
    torch.cuda.synchronize()
    assert torch.all(O3.view(torch.int16) == 0)
    assert torch.allclose(L3, s[None, :, None].expand(B, H, ql), rtol=0, atol=1e-5)


def test_sinks_binding_checks():
    import torch
    q = torch.zeros((1, 4, 8, 64), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError):
        fa.train_fwd_dv(q, q, q, sinks=torch.zeros(3, device="cuda:0"))
    with pytest.raises(TypeError):
        fa.train_fwd_dv(q, q, q, sinks=torch.zeros(4, device="cuda:0", dtype=torch.float64))
    with pytest.raises(ValueError):
        fa.train_fwd_dv(q, q, q, sinks=torch.zeros(4))


SPLIT_CASES = [
    # (B, H, Hkv, ql, kl, D, causal, n_split)
    (1, 8, 1, 1, 1100, 128, False, 8),     # the SDPA page's decode shapes (packed GQA decode)
    (1, 16, 2, 1, 9000, 128, False, 32),
    (2, 32, 8, 1, 5000, 64, True, 16),
    (1, 4, 2, 300, 5000, 64, True, 8),     # prefill against a longer cache
    (1, 2, 1, 300, 200, 64, True, 3),      # ql > kl: chunks no row sees (L_c = -inf)
    (1, 2, 1, 257, 1000, 256, False, 4),
    (1, 2, 2, 17, 900, 128, True, 4),
]


@pytest.mark.parametrize("B,H,Hkv,ql,kl,D,causal,n_split", SPLIT_CASES)
def test_sinks_split_kv(B, H, Hkv, ql, kl, D, causal, n_split):
    """Split-KV with sinks: the chunks' merge adds each row's sink once."""
    import torch
    seed = fagen.SEED_BASE + 0xE00 + ql + kl + D + n_split
    q, k, v = _inputs(seed, B, H, Hkv, ql, kl, D, D)
    s = _sinks(seed, H, kl)
    case = f"sinks split {(B, H, Hkv, ql, kl, D, causal, n_split)}"
    print(f"case {case}", flush=True)
    dev = "cuda:0"
    tq, tk, tv = gu.to_dev(q, dev), gu.to_dev(k, dev), gu.to_dev(v, dev)
    ts = torch.from_numpy(s).to(dev)
    O, L = fa.train_fwd_dv(tq, tk, tv, causal=causal, sinks=ts, n_split=n_split)
    O0, L0 = fa.train_fwd_dv(tq, tk, tv, causal=causal, n_split=n_split)
    neg = torch.full((H,), -math.inf, dtype=torch.float32, device=dev)
    On, Ln = fa.train_fwd_dv(tq, tk, tv, causal=causal, sinks=neg, n_split=n_split)
    torch.cuda.synchronize()
    bits = O.view(torch.int16).cpu().numpy().view(np.uint16)
    of, ob, lr = oracle.fwd_dv(q, k, v, None, B, H, Hkv, ql, kl, D, D, 1.0 / math.sqrt(D), causal,
                               sinks=s)
    tol_o, tol_l = gu.tolerances(kl)
    eo, el, rms = gu.compare(gu.widen(bits), L.cpu().numpy(), bits, ob, lr, tol_o, tol_l,
                             label=case, o_ref_f32=of)
    print(f"{case}: dO={eo:.3e} dL={el:.3e} relRMS={rms:.2e}")
    # -inf sinks: the bits of the same split without sinks
    assert torch.equal(On.view(torch.int16), O0.view(torch.int16))
    assert torch.equal(Ln, L0)
    # the sinks moved L (they sit near the rows' key mass)
    assert float((L - L0).abs().max()) > 0.1
