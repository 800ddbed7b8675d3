"""Pins for the CPU oracle (runs without a GPU).

The oracle is pinned to things other than itself: a double-precision
brute force of the textbook definition (tests/brute.py), closed forms (zero
Q, constant V, a hand-worked two-key example), exact special cases (fully
masked rows, kl = 0, zero mask), invariances (mask shift, GQA == repeated
MHA, the causal sentinel falsifier of the method's page, section 6), and
torch's own bf16 rounding. test_oracle_mutants.py plants mistakes in a copy
of the oracle and checks that these pins catch each one.
"""
import math

import numpy as np
import pytest

import fagen
import oracle
from tests import pins


def test_hand_worked_two_keys():
    pins.pin_hand_worked(oracle.fwd)


@pytest.mark.parametrize("D", [4, 8, 64])
@pytest.mark.parametrize("ql,kl", [(1, 1), (5, 7), (7, 5), (16, 16), (33, 17), (17, 33)])
@pytest.mark.parametrize("H,Hkv", [(1, 1), (2, 1), (4, 2), (8, 2)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("masked", [False, True])
def test_matches_f64_brute_force(D, ql, kl, H, Hkv, causal, masked):
    pins.pin_brute_force(oracle.fwd, B=2, H=H, Hkv=Hkv, ql=ql, kl=kl, D=D, causal=causal,
                         masked=masked, seed=ql * 1000 + kl * 10 + D + H)


@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.5])
def test_other_scales_match_brute_force(scale):
    pins.pin_brute_force(oracle.fwd, B=1, H=2, Hkv=1, ql=9, kl=13, D=8, causal=True,
                         masked=True, seed=77, scale=scale)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("ql,kl", [(8, 8), (5, 12), (12, 5)])
def test_zero_q_closed_form(causal, ql, kl):
    pins.pin_zero_q(oracle.fwd, ql=ql, kl=kl, causal=causal)


def test_constant_v_rows_give_that_row():
    pins.pin_constant_v(oracle.fwd)


def test_fully_masked_rows_are_exact():
    pins.pin_fully_masked(oracle.fwd)


def test_kl_zero_gives_empty_rows():
    O, Ob, L = oracle.fwd(np.zeros((1, 2, 3, 8), np.uint16), np.zeros((1, 1, 0, 8), np.uint16),
                          np.zeros((1, 1, 0, 8), np.uint16), None, 1, 2, 1, 3, 0, 8, 0.5, False)
    assert np.all(O == 0) and not np.signbit(O).any()
    assert np.all(np.isneginf(L))


def test_zero_mask_is_bit_identical_to_no_mask():
    pins.pin_zero_mask(oracle.fwd)


def test_mask_shift_invariance():
    pins.pin_mask_shift(oracle.fwd)


def test_causal_sentinel_falsifier():
    pins.pin_causal_sentinel(oracle.fwd)


def test_causal_offset_alignment():
    pins.pin_causal_alignment(oracle.fwd)


def test_gqa_equals_repeated_mha():
    pins.pin_gqa_repeat(oracle.fwd)


def test_rows_api_is_bit_identical_to_full():
    w = fagen.WORKLOADS["d64_mask_b2_h4_q64_k256_causal"]
    inp = fagen.generate(w)
    O, Ob, L = oracle.fwd_workload(w, inp)
    rows = np.array([0, 5, 63, 64, 200, w.B * w.H * w.ql - 1])
    O2, Ob2, L2 = oracle.fwd_workload(w, inp, rows=rows)
    np.testing.assert_array_equal(O.reshape(-1, w.D)[rows], O2)
    np.testing.assert_array_equal(L.reshape(-1)[rows], L2)


def test_thread_count_does_not_change_bits():
    w = fagen.WORKLOADS["d256_gqa_b2_h8kv2_q128_k128_causal"]
    inp = fagen.generate(w)
    O1, _, L1 = oracle.fwd_workload(w, inp, n_threads=1)
    O8, _, L8 = oracle.fwd_workload(w, inp, n_threads=8)
    np.testing.assert_array_equal(O1, O8)
    np.testing.assert_array_equal(L1, L8)


def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    # add exact ties and near-ties around a few bf16 values, and specials
    base = (rng.integers(0, 2**16, size=2000, dtype=np.uint32) << 16)
    extra = np.concatenate([base | 0x8000, base | 0x7FFF, base | 0x8001, base])
    bits = np.concatenate([bits, extra, np.array([0x7F800000, 0xFF800000, 0, 0x80000000,
                                                  0x7F7FFFFF, 0x7F7F8000], np.uint32)])
    x = bits.view(np.float32)
    finite = ~np.isnan(x)
    x = x[finite]
    ours = oracle.round_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_rejects_bad_head_grouping():
    with pytest.raises(ValueError):
        oracle.fwd(np.zeros((1, 3, 2, 4), np.uint16), np.zeros((1, 2, 2, 4), np.uint16),
                   np.zeros((1, 2, 2, 4), np.uint16), None, 1, 3, 2, 2, 2, 4, 1.0, False)


def test_workload_outputs_are_finite_and_sane():
    """Every workload small enough for the oracle: L finite except fully masked
    rows, |O| bounded by max |V| of the head (O is a convex combination)."""
    for name in ["d64_b1_h2_q64_k64", "d256_gqa_b2_h8kv2_q128_k128_causal",
                 "d64_mask_b2_h4_q64_k256_causal"]:
        w = fagen.WORKLOADS[name]
        inp = fagen.generate(w)
        O, Ob, L = oracle.fwd_workload(w, inp)
        v = oracle.widen_bf16(inp["v"])
        assert np.abs(O).max() <= np.abs(v).max() * (1 + 1e-6)
        if inp["mask"] is None:
            assert np.isfinite(L).all()
        else:
            full = np.isneginf(inp["mask"]).all(-1)
            assert np.isneginf(L[full]).all() and np.isfinite(L[~full]).all()
            assert math.isclose(full.sum(), w.B * w.H * w.mask_full_rows)


def test_dominant_key_one_hot():
    pins.pin_dominant_key(oracle.fwd)


# ---- sliding window (the method page, section 7) ----

@pytest.mark.parametrize("D", [4, 8])
@pytest.mark.parametrize("ql,kl", [(1, 1), (16, 16), (7, 19), (19, 7), (33, 33)])
@pytest.mark.parametrize("window", [0, 1, 5, 16, 40])
@pytest.mark.parametrize("masked", [False, True])
def test_window_matches_f64_brute_force(D, ql, kl, window, masked):
    pins.pin_brute_force(oracle.fwd, B=1, H=4, Hkv=2, ql=ql, kl=kl, D=D, causal=True,
                         masked=masked, seed=ql * 97 + kl * 7 + window, window=window)


def test_window_is_the_page_mask():
    pins.pin_window_is_the_page_mask(oracle.fwd)


def test_window_alignment():
    pins.pin_window_alignment(oracle.fwd)


def test_window_zero_closed_form():
    pins.pin_window_zero(oracle.fwd)


def test_window_wider_than_rows_is_causal():
    pins.pin_window_wide_is_causal(oracle.fwd)


def test_window_rows_match_full():
    B, H, Hkv, ql, kl, D = 2, 4, 2, 21, 30, 8
    q, k, v = pins._inputs(81, B, H, Hkv, ql, kl, D)
    full = oracle.fwd(q, k, v, None, B, H, Hkv, ql, kl, D, 0.3, True, window=6)
    rows = np.array([0, 5, 20, 21, 100, B * H * ql - 1], np.int64)
    part = oracle.fwd_rows(q, k, v, None, B, H, Hkv, ql, kl, D, 0.3, True, rows, window=6)
    assert np.array_equal(part[0], full[0].reshape(-1, D)[rows])
    assert np.array_equal(part[2], full[2].reshape(-1)[rows])


def test_window_negative_is_rejected():
    q, k, v = pins._inputs(82, 1, 1, 1, 4, 4, 8)
    with pytest.raises(ValueError):
        oracle.fwd(q, k, v, None, 1, 1, 1, 4, 4, 8, 0.3, True, window=-1)


@pytest.mark.parametrize("D,Dv", [(8, 24), (24, 8), (96, 64), (192, 128), (64, 64)])
@pytest.mark.parametrize("causal,masked,window", [(False, False, None), (True, True, None),
                                                  (True, False, 4)])
def test_value_width_matches_f64_brute_force(D, Dv, causal, masked, window):
    """Dv != D (keys of one width, values of another) against the f64
    textbook definition."""
    pins.pin_brute_force_dv(oracle.fwd_dv, 2, 4, 2, 13, 19, D, Dv, causal, masked,
                            seed=D * 7 + Dv, window=window)


def test_value_width_equal_is_the_plain_forward():
    q, k, v = pins._inputs(91, 1, 2, 1, 9, 14, 16)
    a = oracle.fwd(q, k, v, None, 1, 2, 1, 9, 14, 16, 0.3, True)
    b = oracle.fwd_dv(q, k, v, None, 1, 2, 1, 9, 14, 16, 16, 0.3, True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("name,pin", pins.SINK_PINS, ids=[n for n, _ in pins.SINK_PINS])
def test_sinks_pins(name, pin):
    """Per-head sink logits (one more softmax term with a zero value): closed
    forms and the f64 brute force of that definition."""
    pin(oracle.fwd_dv)
