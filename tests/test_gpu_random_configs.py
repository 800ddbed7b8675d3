"""Seeded random configurations of the forward, every option through the one
entry point that takes them all (fa_train_fwd_dv), against the oracle (marked
gpu).

Each case draws, from its own seed: a (key, value) head-dim pair of the
kernels, the batch, the kv heads and the GQA group, the query and key counts
(ragged, sometimes one query row, sometimes no key), the scale, and one of: no
mask, the causal rule, a sliding window, a boolean, f32 or bf16 mask (dense or
broadcast over batch and heads), with or without split-KV where it applies
(equal base widths, no mask or window), with or without sinks, on contiguous
tensors or on transposed views of [B, L, H, D]. The oracle is
fa_oracle_fwd_general / fa_oracle_fwd_sinks on the same bf16 inputs; bounds
as in the other forward tests (gpu_util.compare: 5e-3 / 3e-3 up to 256 keys,
1e-2 beyond, the bf16 step rule, exact empty rows).
"""
import math

import numpy as np
import pytest

import fagen
import oracle
import flash_attention_forward_fa_amd as fa
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

PAIRS = [(64, 64), (80, 80), (96, 96), (96, 64), (128, 128), (192, 192), (192, 128),
         (256, 256)]
N_CASES = 64


def _draw(i):
    """The configuration of case i (a pure function of i)."""
    r = np.random.default_rng(0xC0FFEE + 7919 * i)
    # (the equal base widths, which also take split-KV, half of the time)
    base = [p for p in PAIRS if p[0] == p[1] and p[0] in (64, 128, 256)]
    D, Dv = (base[int(r.integers(len(base)))] if r.random() < 0.5
             else PAIRS[int(r.integers(len(PAIRS)))])
    B = int(r.integers(1, 3))
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 4]))
    ql = int(r.choice([1, int(r.integers(2, 17)), int(r.integers(17, 300))], p=[0.2, 0.25, 0.55]))
    kl = int(r.choice([0, int(r.integers(1, 200)), int(r.integers(200, 1400))], p=[0.05, 0.35,
                                                                                     0.6]))
    scale = float(1.0 / math.sqrt(D) if r.random() < 0.6 else r.uniform(0.05, 0.5))
    kind = str(r.choice(["none", "causal", "window", "bool", "f32", "bf16"]))
    window = int(r.integers(0, 300)) if kind == "window" else None
    bshape = (int(r.choice([1, B])), int(r.choice([1, Hkv * G])))
    sinks = bool(r.random() < 0.4)
    views = bool(r.random() < 0.3)
    split_ok = D == Dv and D in (64, 128, 256) and kind in ("none", "causal")
    n_split = int(r.choice([1, 3, 8, 16])) if split_ok and r.random() < 0.7 else 0
    return dict(D=D, Dv=Dv, B=B, Hkv=Hkv, H=Hkv * G, ql=ql, kl=kl, scale=scale, kind=kind,
                window=window, bshape=bshape, sinks=sinks, views=views, n_split=n_split)


def _mask(c, seed):
    """(torch mask for the call or None, f32 oracle mask [B, H, ql, kl] or None)."""
    import torch
    kind, (mb, mh), B, H, ql, kl = c["kind"], c["bshape"], c["B"], c["H"], c["ql"], c["kl"]
    if kind not in ("bool", "f32", "bf16"):
        return None, None
    if kind == "bool":
        add, _ = fagen.mask_f32(seed, mb, mh, ql, kl, p_masked=0.3,
                                n_full_rows=1 if ql >= 4 else 0)
        t = torch.from_numpy(add == 0.0)
    else:
        # finite additive values (bf16-exact, so that the bf16 mask is the same
        # mask) with some hidden keys
        vals = fagen.bf16_bits_to_f32(fagen.normal_bf16(seed, fagen.STREAM_MASK, (mb, mh, ql, kl)))
        hid, _ = fagen.mask_f32(seed + 1, mb, mh, ql, kl, p_masked=0.1, n_full_rows=0)
        add = (vals + hid).astype(np.float32)
        t = torch.from_numpy(add)
        if kind == "bf16":
            t = t.to(torch.bfloat16)
    ref = np.ascontiguousarray(np.broadcast_to(add, (B, H, ql, kl)), dtype=np.float32)
    return t.to("cuda:0"), ref


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_config_matches_oracle(i):
    import torch
    c = _draw(i)
    B, H, Hkv, ql, kl, D, Dv = c["B"], c["H"], c["Hkv"], c["ql"], c["kl"], c["D"], c["Dv"]
    causal = c["kind"] in ("causal", "window")
    print(f"case random {i}: {c}", flush=True)
    seed = fagen.SEED_BASE + 0x7000 + i
    q = fagen.normal_bf16(seed, fagen.STREAM_Q, (B, H, ql, D))
    k = fagen.normal_bf16(seed, fagen.STREAM_K, (B, Hkv, kl, D))
    v = fagen.normal_bf16(seed, fagen.STREAM_V, (B, Hkv, kl, Dv))
    s = None
    if c["sinks"]:
        z = fagen.bf16_bits_to_f32(fagen.normal_bf16(seed, 5, (H,), sigma=2.0))
        s = (np.float32(math.log(max(kl, 1))) + z).astype(np.float32)
    dev = "cuda:0"
    tq, tk, tv = gu.to_dev(q, dev), gu.to_dev(k, dev), gu.to_dev(v, dev)
    if c["views"]:
        tq = tq.transpose(1, 2).contiguous().transpose(1, 2)
        tk = tk.transpose(1, 2).contiguous().transpose(1, 2)
        tv = tv.transpose(1, 2).contiguous().transpose(1, 2)
    tm, ref_mask = _mask(c, seed)
    O, L = fa.train_fwd_dv(tq, tk, tv, mask=tm, scale=c["scale"], causal=causal,
                           window=c["window"],
                           sinks=None if s is None else torch.from_numpy(s).to(dev),
                           n_split=c["n_split"])
    torch.cuda.synchronize()
    bits = O.view(torch.int16).cpu().numpy().view(np.uint16)
    of, ob, lr = oracle.fwd_dv(q, k, v, ref_mask, B, H, Hkv, ql, kl, D, Dv, c["scale"], causal,
                               window=c["window"], sinks=s)
    tol_o, tol_l = gu.tolerances(kl)
    eo, el, rms = gu.compare(gu.widen(bits), L.cpu().numpy(), bits, ob, lr, tol_o, tol_l,
                             label=f"random {i}", o_ref_f32=of)
    print(f"random {i}: dO={eo:.3e} dL={el:.3e} relRMS={rms:.2e}")


def test_draws_cover_every_option():
    """The seeded draws include every pair, mask kind, split, sinks and views."""
    cs = [_draw(i) for i in range(N_CASES)]
    assert {(c["D"], c["Dv"]) for c in cs} == set(PAIRS)
    assert {c["kind"] for c in cs} == {"none", "causal", "window", "bool", "f32", "bf16"}
    assert any(c["n_split"] > 0 for c in cs) and any(c["sinks"] for c in cs)
    assert any(c["views"] for c in cs) and any(c["ql"] == 1 for c in cs)
    assert any(c["kl"] == 0 for c in cs)
    assert any(c["bshape"] != (c["B"], c["H"]) for c in cs if c["kind"] in ("bool", "f32", "bf16"))
