"""fa_train_fwd_split_noalloc, the entry point that allocates nothing (its
split-KV partials live in the library's per-GPU scratch), against the
existing split-KV entry point with a caller workspace: called through the C
ABI twice in a row, the second call smaller, each bit for bit equal to
fa_train_fwd_split on the same inputs and within the oracle's bounds."""
import numpy as np
import pytest

import fagen
import oracle
import flash_attention_forward_fa_amd as fa
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CALLS = [
    # (B, H, Hkv, ql, kl, D, causal, n_split): the first call larger
    (2, 8, 2, 200, 3000, 128, True, 8),
    (1, 4, 1, 1, 1500, 64, False, 5),
]


def _both(w, inp, n_split):
    import torch
    dev = "cuda:0"
    q, k, v = (gu.to_dev(inp[n], dev) for n in ("q", "k", "v"))
    s = torch.cuda.current_stream().cuda_stream
    O1 = torch.full_like(q, float("nan"))
    L1 = torch.full((w.B, w.H, w.ql), float("nan"), device=dev)
    O2, L2 = torch.empty_like(O1), torch.empty_like(L1)
    need = fa.fa_train_fwd_split_workspace(w.B, w.H, w.ql, w.D, n_split)
    assert 0 < need <= fa.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    st = fa.fa_train_fwd_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), w.B, w.H, w.Hkv,
                                       w.ql, w.kl, w.D, w.scale, w.causal, n_split, O1.data_ptr(),
                                       L1.data_ptr(), s)
    assert st == 0, fa.status_string(st)
    st = fa.fa_train_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), w.B, w.H, w.Hkv, w.ql,
                               w.kl, w.D, w.scale, w.causal, n_split, ws.data_ptr(), need,
                               O2.data_ptr(), L2.data_ptr(), s)
    assert st == 0, fa.status_string(st)
    torch.cuda.synchronize()
    b = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    return b(O1), L1.cpu().numpy(), b(O2), L2.cpu().numpy()


def test_noalloc_matches_split_on_two_calls():
    for i, (B, H, Hkv, ql, kl, D, causal, n_split) in enumerate(CALLS):
        w = fagen.Workload("noalloc", B, H, Hkv, ql, kl, D, causal, seed_offset=9900 + i)
        print(f"case noalloc call {i}: {w}", flush=True)
        inp = fagen.generate(w)
        o1, l1, o2, l2 = _both(w, inp, n_split)
        assert np.array_equal(o1, o2), f"call {i}: O differs from fa_train_fwd_split"
        assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32)), f"call {i}: L differs"
        of, ob, lr = oracle.fwd_workload(w, inp)
        tol_o, tol_l = gu.tolerances(kl)
        eo, el, _ = gu.compare(gu.widen(o1), l1, o1, ob, lr, tol_o, tol_l, f"noalloc call {i}", o_ref_f32=of)
        print(f"noalloc call {i}: bit-equal to the workspace call; dO={eo:.3e} dL={el:.3e}",
              flush=True)


def test_noalloc_refuses_more_than_its_scratch():
    import torch
    q = torch.zeros(4, 32, 512, 128, dtype=torch.bfloat16, device="cuda:0")
    k = torch.zeros(4, 8, 4096, 128, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(fa.FAError) as e:
        fa.train_fwd_split_noalloc(q, k, k, 8)
    assert e.value.status == 14
