"""GPU parity of the backward with attention sinks (fa_train_bwd_sinks) against
the oracle: dQ, dK, dV from the sink-aware L (the bounds of test_gpu_bwd.py),
and each head's sink gradient against oracle.bwd_sinks.

Bound of the sink gradient: dsink_h = -sum_i p_i D_i sums one term per row of
the head, p_i = exp(sink_h - L_i). On the GPU, D_i comes from a bf16 O (the GPU
forward's; in the random cases the oracle's, rounded) (one rounding of each O element, a relative 2^-9) and L_i from its
own logsumexp; each term can move by about 2^-8 (4e-3) of sum_d |O_id dO_id|
times p_i, so the bound is 5e-3 times sum_i p_i sum_d |O_id dO_id| (oracle
values), plus 1e-6. (Measured: at most 3% of the bound.)"""
import math

import numpy as np
import pytest

import fagen
import oracle
from tests import gpu_util as gu
from tests.test_gpu_bwd import check_grads

pytestmark = pytest.mark.gpu

NEG = -np.inf
CASES = [
    # name, B, H, Hkv, ql, kl, D, causal, window, mask kind, sinks
    ("d64_causal_gqa", 2, 4, 2, 77, 130, 64, True, None, None, [0.5, -1.0, 2.0, NEG]),
    ("d128_noncausal", 1, 4, 1, 96, 70, 128, False, None, None, [1.0, 0.0, -0.5, 3.0]),
    ("d256_causal_gqa", 1, 4, 2, 200, 200, 256, True, None, None, [-2.0, 0.7, 1.3, 0.0]),
    ("d64_window", 1, 2, 1, 150, 150, 64, True, 40, None, [0.3, -0.8]),
    ("d64_masked_empty_rows", 2, 2, 2, 64, 96, 64, False, None, "rows", [0.5, 1.5]),
    ("d64_ql_gt_kl", 1, 2, 2, 300, 100, 64, True, None, None, [4.0, -3.0]),
]


def _inputs(seed, B, H, Hkv, ql, kl, D, mask_kind):
    q = fagen.normal_bf16(seed, 0, (B, H, ql, D))
    k = fagen.normal_bf16(seed, 1, (B, Hkv, kl, D))
    v = fagen.normal_bf16(seed, 2, (B, Hkv, kl, D))
    dO = fagen.normal_bf16(seed, 6, (B, H, ql, D))
    mask = None
    if mask_kind == "rows":
        mask, _ = fagen.mask_f32(seed, B, H, ql, kl, 0.1, 2)
    return q, k, v, dO, mask


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_with_sinks_matches_oracle(case):
    _run(case, fagen.SEED_BASE + 8100 + CASES.index(case))


def _run(case, seed, shared_o=False):
    """shared_o: both backwards read D from the oracle's forward O rounded to
    bf16 (fa_oracle_bwd_given_o), instead of the GPU backward reading the
    GPU forward's O: with one or two visible keys dP - D cancels almost to
    nothing, and the rounding of O alone then moves dQ and dK by more than
    the RMS bound."""
    import torch
    import flash_attention_forward_fa_amd as fa
    name, B, H, Hkv, ql, kl, D, causal, window, mask_kind, sinks = case
    print(f"case bwd-sinks {name}: B{B} H{H}/{Hkv} ql{ql} kl{kl} D{D} causal={causal} "
          f"window={window} mask={mask_kind} sinks={sinks}", flush=True)
    q, k, v, dO, mask = _inputs(seed, B, H, Hkv, ql, kl, D, mask_kind)
    s = np.asarray(sinks, np.float32)
    scale = 1.0 / math.sqrt(D)
    dev = "cuda:0"
    qd, kd, vd, gd = (gu.to_dev(x, dev) for x in (q, k, v, dO))
    md = None if mask is None else gu.to_dev(mask, dev)
    sd = torch.from_numpy(s).to(dev)
    O, L = fa.train_fwd_dv(qd, kd, vd, mask=md, scale=scale, causal=causal, window=window,
                           sinks=sd)
    Oo, Ob, Lo = oracle.fwd_dv(q, k, v, mask, B, H, Hkv, ql, kl, D, D, scale, causal,
                               window=window, sinks=s)
    if shared_o:
        O.copy_(gu.to_dev(Ob, dev))
    dQ, dK, dV, dS = fa.train_bwd_sinks(qd, kd, vd, O, L, gd, sd, mask=md, scale=scale,
                                        causal=causal, window=window)
    dS2 = fa.train_bwd_sinks(qd, kd, vd, O, L, gd, sd, mask=md, scale=scale, causal=causal,
                             window=window)[3]
    torch.cuda.synchronize()
    got = [gu.widen(t.view(torch.int16).cpu().numpy().view(np.uint16)) for t in (dQ, dK, dV)]
    ref = oracle.bwd(q, k, v, mask, Lo, dO, B, H, Hkv, ql, kl, D, scale, causal, window=window,
                     O=Ob if shared_o else None)
    check_grads(name, got, ref)
    ds_ref = oracle.bwd_sinks(q, k, v, mask, Lo, dO, B, H, Hkv, ql, kl, D, scale, causal, s,
                              window=window)
    ds = dS.cpu().numpy()
    assert np.array_equal(ds, dS2.cpu().numpy()), f"{name}: dsinks differ between two calls"
    g = gu.widen(dO).reshape(B, H, ql, D).astype(np.float64)
    with np.errstate(invalid="ignore"):
        p = np.where(np.isneginf(s)[None, :, None], 0.0,
                     np.exp(s.astype(np.float64)[None, :, None] - Lo.astype(np.float64)))
    scale_h = (p * np.abs(Oo.astype(np.float64) * g).sum(-1)).sum(axis=(0, 2))
    bound = 5e-3 * scale_h + 1e-6
    err = np.abs(ds.astype(np.float64) - ds_ref)
    print(f"bwd-sinks {name}: dsinks {ds} oracle {ds_ref} err {err.max():.3e} "
          f"bound {bound.min():.3e}..{bound.max():.3e}", flush=True)
    assert np.all(err <= bound), f"{name}: dsinks error {err} > {bound}"
    assert np.all(ds[np.isneginf(s)] == 0), f"{name}: a -inf sink has a nonzero gradient"


def test_minus_inf_sinks_equal_the_backward_without_sinks():
    """Sinks of -inf: the forward is the plain one bit for bit, so the gradients
    equal train_bwd_strided's bits and every sink gradient is exactly 0."""
    import torch
    import flash_attention_forward_fa_amd as fa
    B, H, Hkv, ql, kl, D = 1, 4, 2, 130, 130, 64
    print("case bwd-sinks -inf", flush=True)
    q, k, v, dO, _ = _inputs(fagen.SEED_BASE + 8150, B, H, Hkv, ql, kl, D, None)
    dev = "cuda:0"
    qd, kd, vd, gd = (gu.to_dev(x, dev) for x in (q, k, v, dO))
    sd = torch.full((H,), -math.inf, device=dev)
    O, L = fa.train_fwd_dv(qd, kd, vd, causal=True, sinks=sd)
    a = fa.train_bwd_sinks(qd, kd, vd, O, L, gd, sd, causal=True)
    b = fa.train_bwd_strided(qd, kd, vd, O, L, gd, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a[:3], b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert torch.all(a[3] == 0)


def test_sink_gradient_written_without_rows():
    """batch * ql = 0: every head's sink gradient is written (0), over a
    NaN-filled buffer."""
    import torch
    import flash_attention_forward_fa_amd as fa
    print("case bwd-sinks no rows", flush=True)
    dev = "cuda:0"
    H, Hkv, kl, D = 4, 2, 64, 64
    k = torch.zeros(1, Hkv, kl, D, dtype=torch.bfloat16, device=dev)
    q = torch.zeros(1, H, 0, D, dtype=torch.bfloat16, device=dev)
    L = torch.zeros(1, H, 0, device=dev)
    dK, dV = torch.empty_like(k), torch.empty_like(k)
    sinks = torch.ones(H, device=dev)
    ds = torch.full((H,), float("nan"), device=dev)
    st = fa.fa_train_bwd_sinks(0, k.data_ptr(), k.data_ptr(), 0, 0, 0, None, None, 0, 0, None, 1,
                               H, Hkv, 0, kl, D, 0.125, 1, -1, sinks.data_ptr(), 0,
                               dK.data_ptr(), dV.data_ptr(), ds.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    assert st == 0, fa.status_string(st)
    torch.cuda.synchronize()
    assert torch.all(ds == 0)


N_RANDOM = 16
# one-key draws (kl = 1), where dP - D nearly cancels
ONE_KEY_SEEDS = (366, 554)


def _draw(i):
    """Configuration of random case i (a pure function of i): head dim, batch,
    GQA, ragged ql and kl (ql > kl too), causal / window / none, and sinks near
    the log of a row's key count (some -inf)."""
    r = np.random.default_rng(0x51F7 + 7919 * i)
    D = int(r.choice([64, 128, 256]))
    B = int(r.integers(1, 3))
    Hkv = int(r.choice([1, 2]))
    H = Hkv * int(r.choice([1, 2, 4]))
    ql = int(r.choice([1, int(r.integers(2, 70)), int(r.integers(70, 300))], p=[0.1, 0.3, 0.6]))
    kl = int(r.choice([int(r.integers(1, 60)), int(r.integers(60, 400))], p=[0.25, 0.75]))
    kind = str(r.choice(["none", "causal", "window"]))
    window = int(r.integers(0, 80)) if kind == "window" else None
    sinks = (math.log(max(kl, 1)) + 2.0 * r.standard_normal(H)).astype(np.float32)
    sinks[r.random(H) < 0.15] = -np.inf
    return dict(D=D, B=B, Hkv=Hkv, H=H, ql=ql, kl=kl, causal=kind != "none", window=window,
                sinks=sinks)


@pytest.mark.parametrize("i", list(range(N_RANDOM)) + list(ONE_KEY_SEEDS))
def test_random_backward_with_sinks_matches_oracle(i):
    c = _draw(i)
    case = (f"random{i}", c["B"], c["H"], c["Hkv"], c["ql"], c["kl"], c["D"], c["causal"],
            c["window"], None, list(c["sinks"]))
    _run(case, fagen.SEED_BASE + 8200 + i, shared_o=True)
