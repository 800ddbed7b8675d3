"""The backward uses dQ's own memory as scratch: a first launch stores each
query row's L log2(e) and D there, the dK/dV launch reads them, and the dQ
launch reads its rows' values before it overwrites the rows. These tests fill
the output buffers with NaN before the call and check that nothing of the
prior contents survives: the gradients are bit-identical to those of a call
into fresh buffers, and rows without visible keys get exact zeros."""
import math

import numpy as np
import pytest

import fagen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, H, Hkv, ql, kl, D, causal
    ("ragged_gqa_d64", 2, 4, 2, 77, 130, 64, True),
    ("ragged_gqa_d128", 1, 4, 1, 150, 70, 128, True),
    ("ragged_gqa_d256", 1, 4, 2, 90, 200, 256, False),
    ("ql_gt_kl_d64", 1, 2, 2, 200, 40, 64, True),
    ("no_keys_d64", 1, 2, 1, 33, 0, 64, False),
]


def _nan_like(t):
    import torch
    out = torch.empty_like(t)
    out.view(torch.int16).fill_(-1)  # 0xFFFF: a bf16 NaN
    return out


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_overwrites_prefilled_outputs(case):
    import torch
    import flash_attention_forward_fa_amd as fa
    name, B, H, Hkv, ql, kl, D, causal = case
    print(f"case bwd-scratch {name}: B{B} H{H}/{Hkv} ql{ql} kl{kl} D{D} causal={causal}",
          flush=True)
    seed = fagen.SEED_BASE + 7900 + CASES.index(case)
    dev = "cuda:0"
    q = gu.to_dev(fagen.normal_bf16(seed, 0, (B, H, ql, D)), dev)
    k = gu.to_dev(fagen.normal_bf16(seed, 1, (B, Hkv, kl, D)), dev)
    v = gu.to_dev(fagen.normal_bf16(seed, 2, (B, Hkv, kl, D)), dev)
    dO = gu.to_dev(fagen.normal_bf16(seed, 6, (B, H, ql, D)), dev)
    scale = 1.0 / math.sqrt(D)
    O, L = fa.train_fwd(q, k, v, scale=scale, causal=causal)
    ref = fa.train_bwd(q, k, v, O, L, dO, scale=scale, causal=causal)
    dQ, dK, dV = _nan_like(q), _nan_like(k), _nan_like(v)
    s = torch.cuda.current_stream()
    st = fa.fa_train_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), 0, O.data_ptr(),
                         L.data_ptr(), dO.data_ptr(), B, H, Hkv, ql, kl, D, scale, causal,
                         dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(), s.cuda_stream)
    assert st == 0, fa.status_string(st)
    torch.cuda.synchronize()
    for tname, got, want in zip(("dQ", "dK", "dV"), (dQ, dK, dV), ref):
        g = got.view(torch.int16).cpu().numpy()
        w = want.view(torch.int16).cpu().numpy()
        assert not np.isnan(gu.widen(g.view(np.uint16))).any(), f"{name}: NaN left in {tname}"
        assert np.array_equal(g, w), f"{name}: {tname} differs from a call into fresh buffers"
    # rows that see no key: L = -inf, and their dQ rows are exact zeros
    Lh = L.cpu().numpy()
    empty = np.isneginf(Lh)
    if kl == 0:
        assert empty.all()
    if empty.any():
        rows = dQ.view(torch.int16).cpu().numpy()[empty]
        assert (rows == 0).all(), f"{name}: dQ of rows with no visible key is not +0"
