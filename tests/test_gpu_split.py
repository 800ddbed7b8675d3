"""GPU parity of the split-KV forward (fa_train_fwd_split) against the CPU oracle
(marked gpu): the same forward definition, computed as key chunks whose
partial results are merged through their logsumexps. Bounds as for the plain
forward (O <= 5e-3 and L <= 3e-3 while kl <= 256, 1e-2 beyond); rows with no
visible key exactly O = +0, L = -inf.
"""
import numpy as np
import pytest

import fagen
import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def run_split(inp, w, n_split, workspace=None, scale=None):
    import torch
    import flash_attention_forward_fa_amd as fa
    q, k, v = (gu.to_dev(inp[n], "cuda:0") for n in ("q", "k", "v"))
    O, L = fa.train_fwd_split(q, k, v, n_split, scale=w.scale if scale is None else scale,
                              causal=w.causal, workspace=workspace)
    torch.cuda.synchronize()
    bits = O.view(torch.int16).cpu().numpy().view(np.uint16)
    return gu.widen(bits), L.cpu().numpy(), bits


CASES = [
    # (B, H, Hkv, ql, kl, D, causal, n_split)
    (1, 4, 1, 300, 5000, 64, True, 8),      # prefill against a longer cache (offset 4700)
    (2, 8, 2, 1, 3000, 128, True, 16),      # decoding one token
    (1, 4, 4, 4, 2100, 64, False, 33),      # a few query rows, ragged chunks
    (1, 2, 1, 257, 1000, 256, False, 4),
    (1, 8, 2, 512, 4096, 128, True, 32),
    (1, 2, 1, 300, 200, 64, True, 3),       # ql > kl: offset 0, early chunks only
    (1, 2, 2, 100, 100, 64, True, 10),      # more chunks than key tiles
    (2, 4, 2, 64, 700, 256, True, 1),       # one chunk
    # at most 16 query rows (the narrow kernels, one 16-row block per wave)
    (1, 16, 1, 1, 2000, 64, False, 8),      # 16 query heads of one kv head, packed
    (1, 2, 2, 16, 900, 64, True, 4),        # 16 rows, causal offset 884
    (1, 2, 2, 17, 900, 128, True, 4),       # 17 rows: the two-block kernel
    (1, 32, 8, 1, 32768, 128, True, 64),    # decoding against a 32k cache
    # chunks of plain tiles (more than 256 keys), compensated where a chunk's
    # rows see 1 to 127 of its keys
    (1, 4, 2, 700, 3000, 64, True, 3),      # ql < kl: chunks before, across, after the diagonal
    (1, 2, 1, 1000, 1000, 128, True, 5),    # ql = kl: the diagonal crosses every chunk
    (2, 4, 4, 300, 2000, 256, False, 6),    # not causal: a short last chunk (2000 - 5 * 384)
]


@pytest.mark.parametrize("D", [64, 128, 256])
def test_split_plain_chunks_redo(D):
    """V times 16 (exact in bf16) at the usual scale: many rows reach
    |O| >= 1, so plain chunks hand them to their compensated redo; every row
    against the oracle."""
    w = fagen.Workload("split_redo", 1, 4, 2, 512, 4000, D, True, seed_offset=9300 + D)
    print(f"case split redo D={D}", flush=True)
    inp = fagen.generate(w)
    vb = np.asarray(inp["v"], np.uint16)
    e = (vb >> 7) & 0xFF
    assert np.all(e < 250)
    inp["v"] = np.where(e != 0, vb + np.uint16(4 << 7), vb).astype(np.uint16)  # exponent + 4
    o, l, bits = run_split(inp, w, 4)
    of, ob, lr = oracle.fwd(inp["q"], inp["k"], inp["v"], None, w.B, w.H, w.Hkv, w.ql, w.kl,
                            w.D, w.scale, w.causal)
    big = int((np.abs(of) >= 1).any(axis=-1).sum())
    eo, el, rms = gu.compare(o, l, bits, ob, lr, 1e-2, 1e-2, f"split redo D={D}", o_ref_f32=of)
    print(f"split redo D={D}: {big} rows with |O| >= 1, dO={eo:.3e} dL={el:.3e} "
          f"relRMS={rms:.2e}")
    assert big > 0 and rms <= 5e-3


@pytest.mark.parametrize("B,H,Hkv,ql,kl,D,causal,n_split", CASES)
def test_split_matches_oracle(B, H, Hkv, ql, kl, D, causal, n_split):
    w = fagen.Workload("split", B, H, Hkv, ql, kl, D, causal,
                       seed_offset=9000 + ql + kl + D + n_split)
    print(f"case split {(B, H, Hkv, ql, kl, D, causal, n_split)}", flush=True)
    inp = fagen.generate(w)
    o, l, bits = run_split(inp, w, n_split)
    of, ob, lr = oracle.fwd_workload(w, inp)
    tol_o, tol_l = gu.tolerances(kl)
    eo, el, rms = gu.compare(o, l, bits, ob, lr, tol_o, tol_l, f"split {B,H,ql,kl,D,n_split}", o_ref_f32=of)
    print(f"split {(B, H, Hkv, ql, kl, D, causal, n_split)}: dO={eo:.3e} dL={el:.3e} "
          f"relRMS={rms:.2e}")
    assert rms <= 5e-3


def test_split_reused_workspace_and_kl_zero():
    """One workspace serves calls of different sizes in a row (its contents on
    entry do not matter); kl = 0 gives empty rows without using it."""
    import torch
    import flash_attention_forward_fa_amd as fa
    big = fagen.Workload("split_big", 1, 4, 2, 128, 3000, 64, True, seed_offset=9100)
    small = fagen.Workload("split_small", 1, 2, 1, 40, 700, 64, True, seed_offset=9101)
    print("case split workspace reuse", flush=True)
    need = fa.fa_train_fwd_split_workspace(1, 4, 128, 64, 12)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda:0")  # NaN-like garbage
    for w in (big, small, big):
        inp = fagen.generate(w)
        o, l, bits = run_split(inp, w, 12, workspace=ws)
        of, ob, lr = oracle.fwd_workload(w, inp)
        gu.compare(o, l, bits, ob, lr, 1e-2, 1e-2, f"split reuse {w.name}", o_ref_f32=of)
    q = torch.randn(1, 2, 5, 64, device="cuda:0").to(torch.bfloat16)
    k = torch.empty(1, 1, 0, 64, device="cuda:0", dtype=torch.bfloat16)
    O, L = fa.train_fwd_split(q, k, k, 4, workspace=torch.empty(0, dtype=torch.uint8,
                                                                 device="cuda:0"))
    torch.cuda.synchronize()
    assert torch.all(O.float() == 0) and torch.all(torch.isneginf(L))


def test_split_long_cache_sampled_rows():
    """Prefill of 512 tokens against a 32k cache (B1, 32 query heads on 8 kv
    heads, head_dim 128, causal offset 32256), 32 chunks, sampled rows."""
    w = fagen.Workload("split_long", 1, 32, 8, 512, 32768, 128, True, seed_offset=9200)
    print("case split long cache", flush=True)
    inp = fagen.generate(w)
    o, l, bits = run_split(inp, w, 32)
    rng = np.random.default_rng(9200)
    rows = np.unique(np.concatenate([np.arange(64), rng.integers(0, w.B * w.H * w.ql, 160),
                                     31 * w.ql + np.arange(w.ql - 32, w.ql)])).astype(np.int64)
    of, ob, lr = oracle.fwd_workload(w, inp, rows=rows)
    o2, l2, b2 = o.reshape(-1, w.D)[rows], l.reshape(-1)[rows], bits.reshape(-1, w.D)[rows]
    eo, el, rms = gu.compare(o2, l2, b2, ob, lr, 1e-2, 1e-2, "split long cache", o_ref_f32=of)
    print(f"split long cache: {rows.size} rows dO={eo:.3e} dL={el:.3e} relRMS={rms:.2e}")
    assert rms <= 1e-2
    assert np.isfinite(o).all() and np.isfinite(l).all()


def test_split_errors_raise_from_binding():
    import torch
    import flash_attention_forward_fa_amd as fa
    q = torch.zeros(1, 1, 4, 64, device="cuda:0", dtype=torch.bfloat16)
    with pytest.raises(fa.FAError) as e:
        fa.train_fwd_split(q, q, q, 0)
    assert e.value.status == 11
    # a workspace too small: refused by the binding, and by the library itself
    small = torch.empty(16, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(ValueError):
        fa.train_fwd_split(q, q, q, 2, workspace=small)
    O, L = torch.empty_like(q), torch.empty(1, 1, 4, device="cuda:0")
    st = fa.fa_train_fwd_split(q.data_ptr(), q.data_ptr(), q.data_ptr(), 1, 1, 1, 4, 4, 64, 0.125,
                               0, 2, small.data_ptr(), 16, O.data_ptr(), L.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    assert st == 11
