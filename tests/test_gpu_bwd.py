"""GPU parity of the backward (fa_train_bwd) against the backward oracle.

The GPU backward consumes the GPU forward's O and L, as a training step
would; the oracle takes the oracle forward's L, as the method page's backward
tests do. dQ, dK and dV (bf16) are compared element by element. Bound: the
page's backward tests use an absolute 5e-3 on their shapes, whose inputs (uniform in
[-0.5, 0)) give gradients well below one. With N(0,1) inputs the gradients
reach 2-5, where one bf16 step of the output alone is 1.6e-2, and dK, dV sum
over every query row of a group. The bound here is 1e-2 times the largest
reference gradient of the tensor (at least 1) for every element, plus a
relative RMS error of at most 4e-3 over the tensor."""
import math

import numpy as np
import pytest

import fagen
import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, H, Hkv, ql, kl, D, causal, mask
    ("page_d64", 1, 1, 1, 32, 32, 64, False, None),
    ("page_d256", 1, 4, 4, 128, 128, 256, False, None),
    ("page_causal", 1, 1, 1, 64, 64, 64, True, None),
    ("page_swa8", 1, 1, 1, 32, 32, 64, False, "swa8"),
    ("page_gqa", 1, 8, 2, 32, 32, 64, False, None),
    ("gqa_causal_d256", 2, 8, 2, 200, 200, 256, True, None),
    ("tails_d64", 2, 4, 2, 77, 301, 64, True, None),
    ("ql_gt_kl_d64", 1, 2, 1, 300, 100, 64, True, None),
    ("masked_rows_d64", 2, 4, 4, 64, 256, 64, True, "random"),
    ("masked_d256", 1, 2, 1, 96, 130, 256, False, "random"),
    ("one_row", 1, 2, 2, 1, 1, 64, True, None),
    ("long_d64", 1, 2, 2, 1024, 1024, 64, True, None),
    ("d128_gqa_causal", 2, 8, 2, 300, 300, 128, True, None),
    ("d128_masked", 1, 2, 1, 96, 200, 128, False, "random"),
    ("d128_long", 1, 2, 1, 1024, 1024, 128, True, None),
    # the SDPA page's gradient check ("nuvec-core 0.3.0", tests/fast.rs, the
    # attention vjp): 4 query heads on 2 kv heads, 40 x 40, head_dim 64, causal
    ("sdpa_page_vjp", 1, 4, 2, 40, 40, 64, True, None),
]


def _mask(kind, seed, B, H, ql, kl):
    if kind is None:
        return None
    if kind == "swa8":  # the page's sliding window: j <= i and j + 8 >= i
        i = np.arange(ql)[:, None]
        j = np.arange(kl)[None, :]
        m = np.where((j <= i) & (j + 8 >= i), 0.0, -np.inf).astype(np.float32)
        return np.broadcast_to(m, (B, H, ql, kl)).copy()
    m, _ = fagen.mask_f32(seed, B, H, ql, kl, 0.1, 2 if ql > 2 else 0)
    return m


def _run_case(name, B, H, Hkv, ql, kl, D, causal, mask_kind, seed_off, window=None):
    import torch
    import flash_attention_forward_fa_amd as fa
    print(f"case bwd {name}: B{B} H{H}/{Hkv} ql{ql} kl{kl} D{D} causal={causal} "
          f"mask={mask_kind}", flush=True)
    seed = fagen.SEED_BASE + 7000 + seed_off
    q = fagen.normal_bf16(seed, 0, (B, H, ql, D))
    k = fagen.normal_bf16(seed, 1, (B, Hkv, kl, D))
    v = fagen.normal_bf16(seed, 2, (B, Hkv, kl, D))
    dO = fagen.normal_bf16(seed, 6, (B, H, ql, D))
    mask = _mask(mask_kind, seed, B, H, ql, kl)
    scale = 1.0 / math.sqrt(D)
    dev = "cuda:0"
    qd, kd, vd, gd = (gu.to_dev(x, dev) for x in (q, k, v, dO))
    md = None if mask is None else gu.to_dev(mask, dev)
    if window is None:
        O, L = fa.train_fwd(qd, kd, vd, mask=md, scale=scale, causal=causal)
        dQ, dK, dV = fa.train_bwd(qd, kd, vd, O, L, gd, mask=md, scale=scale, causal=causal)
    else:
        O, L = fa.train_fwd_swa(qd, kd, vd, window, mask=md, scale=scale)
        dQ, dK, dV = fa.train_bwd_swa(qd, kd, vd, O, L, gd, window, mask=md, scale=scale)
    torch.cuda.synchronize()
    got = [gu.widen(t.view(torch.int16).cpu().numpy().view(np.uint16)) for t in (dQ, dK, dV)]
    _, _, Lr = oracle.fwd(q, k, v, mask, B, H, Hkv, ql, kl, D, scale, causal, window=window)
    ref = oracle.bwd(q, k, v, mask, Lr, dO, B, H, Hkv, ql, kl, D, scale, causal, window=window)
    check_grads(name, got, ref)
    return got, ref


def check_grads(name, got, ref):
    """Element-wise bounds of bf16 gradients against the oracle's f32 ones:
    every element within 1e-2 times the tensor's largest reference gradient
    (at least 1), and a relative RMS error of at most 4e-3. Also printed: the
    largest error beyond half a bf16 step of the reference value (the GPU's
    own output rounding), relative to the tensor's RMS."""
    errs = []
    for tname, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert not np.isnan(g).any(), f"{name}: NaN in {tname}"
        if not r.size:
            continue
        d = np.abs(g - r)
        err = float(d.max())
        bound = 1e-2 * max(1.0, float(np.abs(r).max()))
        ref_rms = float(np.sqrt(np.mean(r.astype(np.float64) ** 2)))
        rms = float(np.sqrt(np.mean(d.astype(np.float64) ** 2)) / max(ref_rms, 1e-2))
        beyond = float((d - 0.5 * gu.bf16_step(np.maximum(np.abs(r), np.abs(g)))).max())
        errs.append((tname, err, bound, rms, beyond / max(ref_rms, 1e-30), ref_rms))
    print(f"bwd {name}: " + ", ".join(
        f"{t} max {e:.2e}/{b:.2e} rms {m:.1e} beyond-half-step {x:.2e}*rms (rms {rr:.2e})"
        for t, e, b, m, x, rr in errs), flush=True)
    for tname, err, bound, rms, _, _ in errs:
        assert err <= bound, f"{name}: {tname} max error {err:.3e} > {bound:.3e}"
        assert rms <= 4e-3, f"{name}: {tname} relative RMS error {rms:.2e}"


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(case):
    _run_case(*case, seed_off=CASES.index(case))


def test_backward_finite_difference_falsifier():
    """The page's falsifier: gradients at the first element of Q, K and V
    against central differences of sum(O * dO) of the float64 forward."""
    from tests.brute import attention_f64
    got, _ = _run_case("fd", 1, 1, 1, 8, 8, 64, False, None, seed_off=99)
    seed = fagen.SEED_BASE + 7000 + 99
    q, k, v, dO = (gu.widen(fagen.normal_bf16(seed, s, (1, 1, 8, 64))).astype(np.float64)
                   for s in (0, 1, 2, 6))
    scale, h = 1.0 / 8.0, 1e-3
    loss = lambda a, b, c: float((attention_f64(a, b, c, None, scale, False)[0] * dO).sum())
    for pos, g in enumerate(got):
        args_p, args_m = [q.copy(), k.copy(), v.copy()], [q.copy(), k.copy(), v.copy()]
        args_p[pos][0, 0, 0, 0] += h
        args_m[pos][0, 0, 0, 0] -= h
        fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert abs(fd - g[0, 0, 0, 0]) <= 5e-2, f"{'QKV'[pos]}: fd {fd:.5f} gpu {g[0,0,0,0]:.5f}"


def test_backward_constant_v_gives_zero_dq_dk():
    """Every V row equal: dQ and dK vanish (dS = 0), dV = P^T dO."""
    import torch
    import flash_attention_forward_fa_amd as fa
    B, H, Hkv, ql, kl, D = 1, 2, 1, 96, 160, 64
    seed = fagen.SEED_BASE + 7500
    q = fagen.normal_bf16(seed, 0, (B, H, ql, D))
    k = fagen.normal_bf16(seed, 1, (B, Hkv, kl, D))
    c = fagen.normal_bf16(seed, 2, (D,))
    v = np.tile(c, B * Hkv * kl).reshape(B, Hkv, kl, D)
    dO = fagen.normal_bf16(seed, 6, (B, H, ql, D))
    dev = "cuda:0"
    qd, kd, vd, gd = (gu.to_dev(x, dev) for x in (q, k, v, dO))
    O, L = fa.train_fwd(qd, kd, vd, causal=True)
    dQ, dK, dV = fa.train_bwd(qd, kd, vd, O, L, gd, causal=True)
    torch.cuda.synchronize()
    # D_i = O_i . dO_i with O = c rounded to bf16 exactly, and dP_ij = dO_i . c
    # in f32: dS is rounding noise
    assert float(dQ.float().abs().max()) <= 2e-3
    assert float(dK.float().abs().max()) <= 2e-3


WINDOW_CASES = [
    # name, B, H, Hkv, ql, kl, D, window, mask
    ("swa_page8", 1, 1, 1, 32, 32, 64, 8, None),       # the page's backward window case
    ("swa_d64", 2, 4, 2, 300, 300, 64, 100, None),
    ("swa_d64_wide", 1, 2, 1, 700, 700, 64, 300, None),
    ("swa_offset", 1, 2, 2, 150, 400, 64, 130, None),
    ("swa_ql_gt_kl", 1, 2, 1, 400, 150, 64, 90, None),
    ("swa_masked", 2, 2, 2, 64, 256, 64, 70, "random"),
    ("swa_d256", 1, 4, 1, 300, 300, 256, 100, None),
    ("swa_d256_gqa", 2, 8, 2, 260, 260, 256, 64, None),
    ("swa_d256_masked", 1, 2, 1, 96, 130, 256, 40, "random"),
    ("swa_zero", 1, 2, 1, 100, 100, 64, 0, None),
    ("swa_d128", 1, 4, 2, 400, 400, 128, 100, None),
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=[c[0] for c in WINDOW_CASES])
def test_window_backward_matches_oracle(case):
    name, B, H, Hkv, ql, kl, D, window, mask = case
    _run_case(name, B, H, Hkv, ql, kl, D, True, mask, seed_off=200 + WINDOW_CASES.index(case),
              window=window)


def test_window_backward_wide_equals_causal_bit_for_bit():
    """A window that hides nothing beyond the causal rule gives the causal
    backward's bits."""
    import torch
    import flash_attention_forward_fa_amd as fa
    for D in (64, 128, 256):
        B, H, Hkv, ql, kl = 1, 4, 2, 300, 340
        seed = fagen.SEED_BASE + 7700 + D
        q, k, v, dO = (gu.to_dev(fagen.normal_bf16(seed, st, shp), "cuda:0") for st, shp in
                       ((0, (B, H, ql, D)), (1, (B, Hkv, kl, D)), (2, (B, Hkv, kl, D)),
                        (6, (B, H, ql, D))))
        print(f"case bwd wide window D={D}", flush=True)
        O, L = fa.train_fwd(q, k, v, causal=True)
        a = fa.train_bwd(q, k, v, O, L, dO, causal=True)
        b = fa.train_bwd_swa(q, k, v, O, L, dO, 10 ** 6)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16))


TRAINING = [
    # workload, kv-head groups (b * Hkv + g) compared in full
    ("d64_b8_h16_q4096_k4096_causal", [0, 127]),
    ("d256_gqa_b2_h16kv4_q8192_k8192_causal", [0]),
]


@pytest.mark.parametrize("name,groups", TRAINING, ids=[t[0] for t in TRAINING])
def test_backward_training_scale_groups(name, groups):
    """The backward of the two training-scale workloads (the ones the bench
    times) with a seeded upstream gradient: every dQ row of the listed kv-head
    groups' query heads and every dK, dV row of those kv heads against the
    oracle, which computes only those groups."""
    import time
    import torch
    import flash_attention_forward_fa_amd as fa
    w = fagen.WORKLOADS[name]
    print(f"case bwd training {name} groups {groups}", flush=True)
    inp = fagen.generate(w)
    dO = fagen.normal_bf16(w.seed, 6, (w.B, w.H, w.ql, w.D))
    dev = "cuda:0"
    qd, kd, vd, gd = (gu.to_dev(x, dev) for x in (inp["q"], inp["k"], inp["v"], dO))
    O, L = fa.train_fwd(qd, kd, vd, scale=w.scale, causal=True)
    dQ, dK, dV = fa.train_bwd(qd, kd, vd, O, L, gd, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    G = w.H // w.Hkv
    bits = lambda t: gu.widen(t.view(torch.int16).cpu().numpy().view(np.uint16))
    got_q, got_k, got_v = [], [], []
    for grp in groups:
        b, g = divmod(grp, w.Hkv)
        got_q.append(bits(dQ[b, g * G:(g + 1) * G]))
        got_k.append(bits(dK[b, g]))
        got_v.append(bits(dV[b, g]))
    del qd, kd, vd, gd, O, dQ, dK, dV
    t0 = time.perf_counter()
    rows = np.concatenate([(divmod(grp, w.Hkv)[0] * w.H + divmod(grp, w.Hkv)[1] * G) * w.ql
                           + np.arange(G * w.ql) for grp in groups]).astype(np.int64)
    _, _, Lr = oracle.fwd_workload(w, inp, rows=rows)
    Lfull = np.zeros((w.B * w.H * w.ql,), np.float32)
    Lfull[rows] = Lr
    ref = oracle.bwd_groups(inp["q"], inp["k"], inp["v"], None, Lfull.reshape(w.B, w.H, w.ql), dO,
                            w.B, w.H, w.Hkv, w.ql, w.kl, w.D, w.scale, True, groups)
    print(f"bwd training {name}: oracle for {len(groups)} group(s) in "
          f"{time.perf_counter() - t0:.1f} s", flush=True)
    got = [np.stack(got_q), np.stack(got_k), np.stack(got_v)]
    check_grads(f"training {name}", got, ref)
