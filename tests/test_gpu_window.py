"""GPU parity of the sliding-window forward (fa_train_fwd_swa) against the CPU
oracle's sliding window, on the same seeded inputs (marked gpu).

The window is the band of the method page's sliding-window test (section 7):
key j visible to row i iff q_abs - window <= j <= q_abs, q_abs = max(kl - ql,
0) + i. Bounds as for the plain forward: O <= 5e-3 and L <= 3e-3 while kl <=
256, 1e-2 beyond; rows with no visible key exactly O = +0, L = -inf.
"""
import numpy as np
import pytest

import fagen
import oracle
from tests import gpu_util as gu
from tests.pins import swa_mask

pytestmark = pytest.mark.gpu


def run_swa(inputs, w, window, dev="cuda:0"):
    import torch
    import flash_attention_forward_fa_amd as fa
    q, k, v = (gu.to_dev(inputs[n], dev) for n in ("q", "k", "v"))
    mask = None if inputs.get("mask") is None else gu.to_dev(inputs["mask"], dev)
    O, L = fa.train_fwd_swa(q, k, v, window, mask=mask, scale=w.scale)
    torch.cuda.synchronize()
    bits = O.view(torch.int16).cpu().numpy().view(np.uint16)
    return gu.widen(bits), L.cpu().numpy(), bits


def test_page_shape_matches_oracle_and_the_page_mask():
    """The page's sliding-window case: B=1, H=2, ql=kl=64, D=64, window 16.
    The native band matches the oracle, and so does the masked forward given
    the page's own 0/-inf mask construction."""
    w = fagen.Workload("swa_page", 1, 2, 2, 64, 64, 64, True, seed_offset=5000)
    print("case swa page shape", flush=True)
    inp = fagen.generate(w)
    o, l, bits = run_swa(inp, w, 16)
    of, ob, lr = oracle.fwd_workload(w, inp, window=16)
    eo, el, _ = gu.compare(o, l, bits, ob, lr, 5e-3, 3e-3, "swa page", o_ref_f32=of)
    print(f"swa page: dO={eo:.3e} dL={el:.3e}")
    inp_m = dict(inp, mask=swa_mask(1, 2, 64, 64, 16))
    o2, l2, b2 = gu.run(inp_m, w.with_(causal=False))
    gu.compare(o2, l2, b2, ob, lr, 5e-3, 3e-3, "page mask through the masked forward", o_ref_f32=of)


WINDOWED = [
    # (B, H, Hkv, ql, kl, D, window, masked)
    (1, 2, 1, 300, 300, 64, 0, False),       # one key per row: O = V[q_abs]
    (2, 4, 2, 333, 333, 64, 100, False),     # every row under 128 keys: compensated
    (1, 2, 1, 700, 700, 64, 200, False),     # plain tiles, skipped tiles, both edges
    (1, 2, 2, 200, 500, 64, 130, False),     # ql < kl: offset 300
    (1, 2, 1, 500, 200, 64, 150, False),     # ql > kl: rows past kl lose keys
    (1, 2, 1, 300, 200, 64, 400, False),     # ql > kl, wide window: mixed launch
    (2, 2, 2, 70, 190, 64, 40, True),        # additive mask on top of the band
    (1, 3, 1, 257, 300, 64, 63, False),
    (1, 4, 1, 300, 300, 256, 64, False),
    (1, 2, 1, 600, 600, 256, 300, False),
    (1, 2, 2, 64, 96, 256, 20, True),
    (1, 1, 1, 300, 40, 256, 10, False),      # ql > kl: rows without any key
    (1, 2, 1, 129, 129, 256, 127, False),
    (1, 2, 1, 500, 500, 128, 150, False),
    (1, 2, 2, 100, 100, 128, 40, True),
]


@pytest.mark.parametrize("B,H,Hkv,ql,kl,D,window,masked", WINDOWED)
def test_windowed_shapes_match_oracle(B, H, Hkv, ql, kl, D, window, masked):
    w = fagen.Workload("swa", B, H, Hkv, ql, kl, D, True,
                       mask_p=0.1 if masked else None, mask_full_rows=2 if masked else 0,
                       seed_offset=5100 + ql * 7 + kl + D + window)
    print(f"case swa {(B, H, Hkv, ql, kl, D, window, masked)}", flush=True)
    inp = fagen.generate(w)
    o, l, bits = run_swa(inp, w, window)
    of, ob, lr = oracle.fwd_workload(w, inp, window=window)
    tol_o, tol_l = gu.tolerances(kl)
    eo, el, _ = gu.compare(o, l, bits, ob, lr, tol_o, tol_l, f"swa {B,H,Hkv,ql,kl,D,window}", o_ref_f32=of)
    print(f"swa {(B, H, Hkv, ql, kl, D, window, masked)}: dO={eo:.3e} dL={el:.3e} "
          f"empty rows={int(np.isneginf(lr).sum())}")
    if window == 0:
        off = max(kl - ql, 0)
        for i in range(min(ql, kl - off)):
            assert np.array_equal(bits[0, :, i], np.broadcast_to(inp["v"][0, 0, off + i],
                                                                 bits[0, :, i].shape))


@pytest.mark.parametrize("D", [64, 128, 256])
def test_wide_window_equals_causal_bit_for_bit(D):
    """A window reaching past every row's first key hides nothing more than
    the causal rule: the window kernel gives the causal kernel's bits."""
    import torch
    import flash_attention_forward_fa_amd as fa
    w = fagen.Workload("swa_wide", 1, 4, 2, 520, 600, D, True, seed_offset=5200 + D)
    print(f"case swa wide D={D}", flush=True)
    inp = fagen.generate(w)
    q, k, v = (gu.to_dev(inp[n], "cuda:0") for n in ("q", "k", "v"))
    Oc, Lc = fa.train_fwd(q, k, v, scale=w.scale, causal=True)
    for window in (599, 600, 10 ** 9):
        Ow, Lw = fa.train_fwd_swa(q, k, v, window, scale=w.scale)
        torch.cuda.synchronize()
        assert torch.equal(Oc.view(torch.int16), Ow.view(torch.int16)), window
        assert torch.equal(Lc, Lw), window


@pytest.mark.parametrize("D", [64, 128, 256])
def test_keys_below_the_window_are_never_seen(D):
    """The page's causal falsifier turned to the window's lower edge: K rows
    below position t are set to 128.0, which would dominate any softmax that
    saw them. Rows whose window starts at or after t are bit-identical to the
    clean run; among the rows that still see keys below t (those whose
    q.128 score is positive dominate) some change."""
    import torch
    import flash_attention_forward_fa_amd as fa
    ql = kl = 640
    window, t = 150, 300
    w = fagen.Workload("swa_sentinel", 1, 2, 1, ql, kl, D, True, seed_offset=5300 + D)
    print(f"case swa sentinel D={D}", flush=True)
    inp = fagen.generate(w)
    kp = inp["k"].copy()
    kp[0, 0, :t] = np.uint16(0x4300)  # 128.0 in bf16
    q, k, v = (gu.to_dev(inp[n], "cuda:0") for n in ("q", "k", "v"))
    a_o, a_l = fa.train_fwd_swa(q, k, v, window, scale=w.scale)
    b_o, b_l = fa.train_fwd_swa(q, gu.to_dev(kp, "cuda:0"), v, window, scale=w.scale)
    torch.cuda.synchronize()
    first_clean = t + window  # q_abs - window >= t
    assert torch.equal(a_o[:, :, first_clean:].view(torch.int16),
                       b_o[:, :, first_clean:].view(torch.int16))
    assert torch.equal(a_l[:, :, first_clean:], b_l[:, :, first_clean:])
    assert not torch.equal(a_l[:, :, first_clean - 64:first_clean],
                           b_l[:, :, first_clean - 64:first_clean])


def _window_rows(w, window, rng):
    rows = set()
    for (b, h) in [(0, 0), (w.B - 1, w.H - 1)]:
        base = (b * w.H + h) * w.ql
        rows.update(base + i for i in range(130))
        for c in (window - 1, window, window + 1, window + 63, window + 64, window + 255,
                  window + 256, w.ql // 2, w.ql - 1):
            rows.add(base + min(max(c, 0), w.ql - 1))
    rows.update(int(r) for r in rng.integers(0, w.B * w.H * w.ql, size=96))
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("name,window", [("d64_b8_h16_q4096_k4096_causal", 1024),
                                         ("d256_gqa_b2_h16kv4_q8192_k8192_causal", 2048)])
def test_training_scale_window_sampled_rows(name, window):
    w = fagen.WORKLOADS[name]
    print(f"case {name} window={window}", flush=True)
    inp = fagen.generate(w)
    o, l, bits = run_swa(inp, w, window)
    rows = _window_rows(w, window, np.random.default_rng(window))
    of, ob, lr = oracle.fwd_workload(w, inp, rows=rows, window=window)
    o2, l2, b2 = o.reshape(-1, w.D)[rows], l.reshape(-1)[rows], bits.reshape(-1, w.D)[rows]
    eo, el, rms = gu.compare(o2, l2, b2, ob, lr, 1e-2, 1e-2, f"{name} window {window}", o_ref_f32=of)
    print(f"{name} window={window}: {rows.size} rows, dO={eo:.3e} dL={el:.3e} relRMS={rms:.2e}")
    assert rms <= 1e-2
    assert np.isfinite(o).all() and np.isfinite(l).all()


def test_window_errors_raise_from_binding():
    import torch
    import flash_attention_forward_fa_amd as fa
    q = torch.zeros(1, 1, 4, 64, device="cuda:0", dtype=torch.bfloat16)
    with pytest.raises(fa.FAError) as e:
        fa.train_fwd_swa(q, q, q, -1)
    assert e.value.status == 9
