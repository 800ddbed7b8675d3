"""GPU tests of independent calls: a call's result does not depend on the
calls before it (a small problem, a larger one, the small one again give
bit-identical results) nor on calls running at the same time on another
stream. Inputs have V scaled by 4 so that many rows reach |O| >= 1 and take
the compensated redo of their query tile."""
import numpy as np
import pytest

import fagen
import oracle
from tests import gpu_util as gu
from tests.test_gpu_parity import _times4

pytestmark = pytest.mark.gpu


def _inputs(w):
    inp = dict(fagen.generate(w))
    inp["v"] = _times4(inp["v"])
    return inp


_keep = []


def _upload(torch, inp):
    t = tuple(gu.to_dev(inp[n], "cuda:0") for n in ("q", "k", "v"))
    _keep.extend(t)  # inputs stay allocated until the streams are synchronised
    return t


def _launch(fa, torch, qkv, w, stream=None):
    q, k, v = qkv
    return fa.train_fwd(q, k, v, scale=w.scale, causal=w.causal, stream=stream)


def _bits(O):
    import torch
    return O.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_calls_are_independent_across_sizes_and_streams(D):
    import torch
    import flash_attention_forward_fa_amd as fa
    small = fagen.Workload("q_small", 1, 2, 1, 300, 300, D, True, seed_offset=4000 + D)
    large = fagen.Workload("q_large", 2, 4, 2, 1100, 1100, D, True, seed_offset=4100 + D)
    print(f"case calls D={D}", flush=True)
    inp_s, inp_l = _inputs(small), _inputs(large)
    dev_s, dev_l = _upload(torch, inp_s), _upload(torch, inp_l)
    torch.cuda.synchronize()

    # small, large, small again on the default stream
    O1, L1 = _launch(fa, torch, dev_s, small)
    O2, L2 = _launch(fa, torch, dev_l, large)
    O3, L3 = _launch(fa, torch, dev_s, small)
    torch.cuda.synchronize()
    for (O, L, w, inp) in ((O1, L1, small, inp_s), (O2, L2, large, inp_l)):
        of, ob, lr = oracle.fwd_workload(w, inp)
        big = int((np.abs(gu.widen(ob)) >= 1).any(axis=-1).sum())
        assert big >= 20, big
        bits = _bits(O)
        gu.compare(gu.widen(bits), L.cpu().numpy(), bits, ob, lr, 1e-2, 1e-2,
                   f"calls {w.name} D={D}", o_ref_f32=of)
    assert np.array_equal(_bits(O1), _bits(O3))
    assert np.array_equal(L1.cpu().numpy().view(np.uint32), L3.cpu().numpy().view(np.uint32))

    # both problems at once on two new streams
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    O4, L4 = _launch(fa, torch, dev_l, large, stream=s1)
    O5, L5 = _launch(fa, torch, dev_s, small, stream=s2)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(O4), _bits(O2))
    assert np.array_equal(L4.cpu().numpy().view(np.uint32), L2.cpu().numpy().view(np.uint32))
    assert np.array_equal(_bits(O5), _bits(O1))
    assert np.array_equal(L5.cpu().numpy().view(np.uint32), L1.cpu().numpy().view(np.uint32))
    _keep.clear()
    print(f"calls D={D}: repeated, resized and concurrent calls bit-identical", flush=True)
