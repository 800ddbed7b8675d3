"""Host-side checks of the binding and the C-ABI library that need no GPU:
every caller-supplied output, lse and workspace tensor is checked (device,
dtype, shape, layout) before its pointer reaches the library, and written
tensors whose strides alias elements are refused (library: FA_ERR_STRIDE;
binding: copied to a layout that does not alias). The library call is
replaced by a stub here, so nothing reaches HIP; GPU residency is decided by
a stand-in for the binding's `_on_gpu`."""
import contextlib

import pytest
import torch

import flash_attention_forward_fa_amd as fa

A = 0x10000  # a 16-byte aligned fake address; never dereferenced


# ---- the C ABI: written tensors whose strides alias elements ----

STRIDED = dict(q=A, q_strides=None, k=A, k_strides=None, v=A, v_strides=None, mask=0,
               mask_dtype=0, mask_strides=None, batch=2, n_heads=4, n_kv_heads=2, ql=8, kl=8,
               head_dim=64, scale=0.125, causal=1, window=-1, n_split=0, workspace=0,
               workspace_bytes=0, O=A, o_strides=None, L=A, stream=0)


@pytest.mark.parametrize("o_strides", [
    (0, 512, 64),            # both batches write the same rows
    (2048, 0, 64),           # every head writes the same rows
    (2048, 512, 32),         # rows shorter than head_dim apart
    (2048, 256, 64),         # heads closer than their 8 rows
    (512, 512, 64),          # batch stride equal to the head stride
])
def test_fwd_strided_refuses_aliasing_output(o_strides):
    args = dict(STRIDED, o_strides=o_strides)
    assert fa.fa_train_fwd_strided(**args) == 13


BWD = dict(q=A, k=A, v=A, O=A, L=A, dO=A, q_strides=None, kv_strides=None, mask=0, mask_dtype=0,
           mask_strides=None, batch=2, n_heads=4, n_kv_heads=2, ql=8, kl=8, head_dim=64,
           scale=0.125, causal=1, window=-1, dQ=A, dK=A, dV=A, stream=0)


@pytest.mark.parametrize("over", [
    dict(kv_strides=(0, 512, 64)),        # K expanded over the batch: dK rows shared
    dict(kv_strides=(1024, 0, 64)),       # expanded over kv heads
    dict(q_strides=(0, 512, 64)),
    dict(q_strides=(2048, 512, 8)),       # rows 8 elements apart, head_dim 64
])
def test_bwd_strided_refuses_aliasing_gradients(over):
    assert fa.fa_train_bwd_strided(**dict(BWD, **over)) == 13


def test_single_batch_or_head_strides_are_free():
    # a dimension of size 1 never aliases, whatever its stride; these layouts
    # pass the stride checks (and then fail on the null workspace for split)
    args = dict(STRIDED, batch=1, o_strides=(0, 512, 64), n_split=2)
    assert fa.fa_train_fwd_strided(**args) == 1
    args = dict(BWD, batch=1, kv_strides=(0, 512, 64), q=0)
    assert fa.fa_train_bwd_strided(**args) == 1


def test_decode_packing_keeps_head_strides_in_range():
    # one query row per head with GQA packs a group's heads as rows of one
    # head; a head stride of 2^31 elements must not be truncated to a 32-bit
    # row stride. The call validates (it fails only on the null workspace of
    # the split path, after the packing decision).
    big = 1 << 31
    args = dict(STRIDED, batch=1, ql=1, q_strides=(4 * big, big, 64),
                o_strides=(4 * big, big, 64), n_split=2)
    assert fa.fa_train_fwd_strided(**args) == 1


# ---- the binding: outputs, lse and workspaces are checked ----

class _Stub:
    """Stands in for the loaded library: records calls, reports success."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def f(*args):
            self.calls.append((name, args))
            return 1 << 20 if name.endswith("_workspace") else 0
        return f


@pytest.fixture
def cpu_as_gpu(monkeypatch):
    """Treat CPU tensors as GPU-resident, except the ones listed in `off`;
    stub the library and torch.cuda's device and stream handling."""
    off = []
    stub = _Stub()
    monkeypatch.setattr(fa, "_on_gpu", lambda t: not any(t is x for x in off))
    monkeypatch.setattr(fa, "lib", lambda: stub)
    monkeypatch.setattr(torch.cuda, "device", lambda d: contextlib.nullcontext())

    class _S:
        cuda_stream = 0
    monkeypatch.setattr(torch.cuda, "current_stream", lambda d=None: _S())
    return off, stub


def _qkv(B=1, H=2, Hkv=1, ql=8, kl=8, D=64):
    q = torch.zeros(B, H, ql, D, dtype=torch.bfloat16)
    k = torch.zeros(B, Hkv, kl, D, dtype=torch.bfloat16)
    return q, k, k.clone()


def _wrappers():
    """(name, call(q, k, v, out, lse, workspace)) for every forward wrapper
    that takes caller outputs."""
    return [
        ("train_fwd", lambda q, k, v, o, l, w: fa.train_fwd(q, k, v, out=o, lse=l)),
        ("train_fwd_swa", lambda q, k, v, o, l, w: fa.train_fwd_swa(q, k, v, 4, out=o, lse=l)),
        ("train_fwd_ex", lambda q, k, v, o, l, w: fa.train_fwd_ex(q, k, v, out=o, lse=l)),
        ("train_fwd_split", lambda q, k, v, o, l, w: fa.train_fwd_split(q, k, v, 2, out=o, lse=l,
                                                                        workspace=w)),
        ("train_fwd_strided", lambda q, k, v, o, l, w: fa.train_fwd_strided(
            q, k, v, out=o, lse=l, n_split=2, workspace=w)),
        ("paged_fwd", lambda q, k, v, o, l, w: fa.paged_fwd(
            q, k, v, torch.zeros(1, 1, dtype=torch.int32), torch.zeros(1, dtype=torch.int32),
            out=o, lse=l, n_split=2, workspace=w)),
    ]


@pytest.mark.parametrize("name,call", _wrappers())
def test_wrappers_accept_valid_outputs(cpu_as_gpu, name, call):
    off, stub = cpu_as_gpu
    q, k, v = _qkv()
    O = torch.empty_like(q)
    L = torch.empty(1, 2, 8)
    ws = torch.empty(1 << 20, dtype=torch.uint8)
    got = call(q, k, v, O, L, ws)
    assert got[0] is O and got[1] is L
    assert stub.calls and stub.calls[-1][0].startswith("fa_")


@pytest.mark.parametrize("name,call", _wrappers())
@pytest.mark.parametrize("bad", ["out_cpu", "out_dtype", "out_shape", "out_layout", "lse_cpu",
                                 "lse_dtype", "lse_shape", "lse_layout", "ws_cpu", "ws_dtype",
                                 "ws_small", "ws_layout"])
def test_wrappers_refuse_bad_outputs(cpu_as_gpu, name, call, bad):
    off, stub = cpu_as_gpu
    q, k, v = _qkv()
    O = torch.empty_like(q)
    L = torch.empty(1, 2, 8)
    ws = torch.empty(1 << 20, dtype=torch.uint8)
    if bad.startswith("ws") and name not in ("train_fwd_split", "train_fwd_strided",
                                             "paged_fwd"):
        pytest.skip("no workspace")
    if bad == "out_cpu":
        off.append(O)
    elif bad == "out_dtype":
        O = O.float()
    elif bad == "out_shape":
        O = torch.empty(1, 2, 7, 64, dtype=torch.bfloat16)
    elif bad == "out_layout":
        # non-contiguous rows for the contiguous entry points; for the strided
        # one a view whose last dimension is not contiguous
        O = torch.empty(1, 2, 64, 8, dtype=torch.bfloat16).transpose(2, 3)
    elif bad == "lse_cpu":
        off.append(L)
    elif bad == "lse_dtype":
        L = L.double()
    elif bad == "lse_shape":
        L = torch.empty(2, 8)
    elif bad == "lse_layout":
        L = torch.empty(1, 8, 2).transpose(1, 2)
    elif bad == "ws_cpu":
        off.append(ws)
    elif bad == "ws_dtype":
        ws = torch.empty(1 << 18, dtype=torch.float32)
    elif bad == "ws_small":
        ws = torch.empty(16, dtype=torch.uint8)
    elif bad == "ws_layout":
        ws = torch.empty(2 << 20, dtype=torch.uint8)[::2]
    with pytest.raises((ValueError, TypeError)):
        call(q, k, v, O, L, ws)
    assert not stub.calls or all(c[0].endswith("_workspace") for c in stub.calls)


def test_strided_wrapper_refuses_aliasing_out(cpu_as_gpu):
    off, stub = cpu_as_gpu
    q, k, v = _qkv(B=2)
    O = torch.empty(1, 2, 8, 64, dtype=torch.bfloat16).expand(2, 2, 8, 64)
    with pytest.raises(ValueError):
        fa.train_fwd_strided(q, k, v, out=O)
    assert not stub.calls


@pytest.mark.parametrize("name", ["train_bwd", "train_bwd_ex", "train_bwd_strided"])
def test_backward_refuses_bad_lse(cpu_as_gpu, name):
    off, stub = cpu_as_gpu
    q, k, v = _qkv()
    f = getattr(fa, name)
    for L in (torch.empty(1, 2, 8, dtype=torch.float64), torch.empty(1, 2, 9)):
        with pytest.raises((ValueError, TypeError)):
            f(q, k, v, q, L, q)
    L = torch.empty(1, 2, 8)
    off.append(L)
    with pytest.raises(ValueError):
        f(q, k, v, q, L, q)
    assert not stub.calls


def test_backward_strided_copies_expanded_inputs(cpu_as_gpu):
    """K and V expanded over the batch (stride 0) would make dK and dV, which
    take K's strides, alias; the binding passes contiguous copies instead."""
    off, stub = cpu_as_gpu
    B, H, Hkv, n, D = 2, 2, 1, 8, 64
    q = torch.zeros(B, H, n, D, dtype=torch.bfloat16)
    k1 = torch.zeros(1, Hkv, n, D, dtype=torch.bfloat16)
    k, v = k1.expand(B, Hkv, n, D), k1.expand(B, Hkv, n, D)
    L = torch.empty(B, H, n)
    dQ, dK, dV = fa.train_bwd_strided(q, k, v, q, L, q)
    name, args = stub.calls[-1]
    assert name == "fa_train_bwd_strided"
    kv_strides = tuple(args[7])
    assert kv_strides[0] == Hkv * n * D
    for t in (dQ, dK, dV):
        assert fa._non_overlapping(t.shape, t.stride())


@pytest.mark.parametrize("shape,strides,ok", [
    ((2, 4, 8, 64), (2048, 512, 64, 1), True),
    ((2, 4, 8, 64), (0, 512, 64, 1), False),
    ((1, 4, 8, 64), (0, 512, 64, 1), True),
    ((2, 4, 8, 64), (64, 128, 512, 1), True),     # [B, L, H, D] viewed as [B, H, L, D]... permuted
    ((2, 4, 8, 64), (4096, 1024, 64, 1), True),   # gaps between heads
    ((2, 4, 8, 64), (2048, 512, 32, 1), False),
    ((2, 4, 8, 64), (2048, 448, 64, 1), False),
])
def test_non_overlapping(shape, strides, ok):
    assert fa._non_overlapping(shape, strides) is ok
