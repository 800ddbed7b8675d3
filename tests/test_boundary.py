"""The C-ABI library: it loads, exports every function include/*.h declares,
and rejects invalid arguments on the host before any HIP call (no GPU needed:
every call here fails validation or is an empty no-op, so nothing is ever
launched)."""
import glob
import math
import os
import re
import subprocess

import pytest

import flash_attention_forward_fa_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for path in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        for m in re.finditer(r"\b([A-Za-z_]\w*)\s*\([^;{)]*\)\s*;", text):
            names.add(m.group(1))
    return names


def test_header_declares_the_entry_points():
    names = _declared_functions()
    assert {"fa_train_fwd", "fa_train_fwd_swa", "fa_train_fwd_ex", "fa_train_fwd_split",
            "fa_train_fwd_split_workspace", "fa_paged_fwd", "fa_train_bwd", "fa_train_bwd_swa",
            "fa_train_bwd_ex", "fa_train_fwd_strided", "fa_train_bwd_strided",
            "fa_train_fwd_dv", "fa_train_bwd_sinks", "fa_status_string"} <= names


def test_library_exports_every_declared_symbol():
    lib = fa.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(lib, name), name


def test_status_strings_cover_all_codes():
    for code in range(0, 15):
        s = fa.status_string(code)
        assert s and s != "unknown status"
    assert fa.status_string(12345) == "unknown status"


A = 0x10000  # a 16-byte aligned fake address; never dereferenced (validation fails first)

GOOD = dict(q=A, k=A, v=A, mask=0, batch=1, n_heads=2, n_kv_heads=1, ql=8, kl=8, head_dim=64,
            scale=0.125, causal=0, O=A, L=A, stream=0)


def _call(**over):
    args = dict(GOOD)
    args.update(over)
    return fa.fa_train_fwd(**args)


@pytest.mark.parametrize("over,code", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(O=0), 1), (dict(L=0), 1),
    (dict(batch=-1), 2), (dict(ql=-1), 2), (dict(kl=-3), 2), (dict(n_heads=0), 2),
    (dict(n_kv_heads=0), 2), (dict(n_heads=3, n_kv_heads=2), 3), (dict(head_dim=72), 4),
    (dict(head_dim=0), 4), (dict(head_dim=112), 4), (dict(scale=math.nan), 5), (dict(scale=math.inf), 5),
    (dict(scale=-math.inf), 5), (dict(q=A + 2), 6), (dict(k=A + 8), 6), (dict(O=A + 4), 6),
    (dict(mask=A + 2), 6), (dict(L=A + 1), 6),
    # (ql = 2: with ql = 1 the GQA heads would be packed into 65536-row heads,
    # a valid size that would reach the launch)
    (dict(batch=65536, n_heads=65536, n_kv_heads=1, ql=2), 7),
])
def test_invalid_arguments_are_rejected(over, code):
    assert _call(**over) == code


@pytest.mark.parametrize("over", [dict(batch=0), dict(ql=0), dict(batch=0, q=0, k=0, v=0, O=0,
                                                                   L=0)])
def test_empty_problems_are_noops(over):
    assert _call(**over) == 0


SWA_GOOD = {k: v for k, v in GOOD.items() if k != "causal"}


def _call_swa(**over):
    args = dict(SWA_GOOD, window=4)
    args.update(over)
    return fa.fa_train_fwd_swa(**args)


@pytest.mark.parametrize("over,code", [
    (dict(window=-1), 9), (dict(window=-(2 ** 31)), 9), (dict(q=0), 1), (dict(v=0), 1),
    (dict(L=0), 1), (dict(kl=-1), 2), (dict(n_heads=3, n_kv_heads=2), 3), (dict(head_dim=72), 4),
    (dict(scale=math.nan), 5), (dict(k=A + 8), 6), (dict(mask=A + 2), 6),
    (dict(batch=65536, n_heads=65536, n_kv_heads=1, ql=1), 7),
])
def test_window_invalid_arguments_are_rejected(over, code):
    assert _call_swa(**over) == code


@pytest.mark.parametrize("over", [dict(batch=0), dict(ql=0, window=0),
                                  dict(ql=0, q=0, k=0, v=0, O=0, L=0, window=2 ** 31 - 1)])
def test_window_empty_problems_are_noops(over):
    assert _call_swa(**over) == 0


EX_GOOD = dict(SWA_GOOD, mask=A, mask_dtype=0, mask_stride_b=0, mask_stride_h=64, causal=1,
               window=-1)


def _call_ex(**over):
    args = dict(EX_GOOD)
    args.update(over)
    return fa.fa_train_fwd_ex(**args)


@pytest.mark.parametrize("over,code", [
    (dict(mask_dtype=3), 10), (dict(mask_dtype=-1), 10), (dict(mask_stride_b=-1), 10),
    (dict(mask_stride_h=-64), 10), (dict(causal=0, window=3), 9), (dict(mask=A + 2), 6),
    (dict(mask=A + 1, mask_dtype=1), 6), (dict(q=0), 1), (dict(head_dim=32), 4),
    (dict(n_heads=3, n_kv_heads=2), 3), (dict(scale=math.inf), 5), (dict(ql=-2), 2),
    (dict(batch=65536, n_heads=65536, n_kv_heads=1, ql=1), 7),
])
def test_ex_invalid_arguments_are_rejected(over, code):
    assert _call_ex(**over) == code


@pytest.mark.parametrize("over", [dict(batch=0), dict(ql=0, mask_dtype=1, mask=A + 2),
                                  dict(batch=0, mask=0, mask_dtype=7, mask_stride_b=-5)])
def test_ex_empty_problems_are_noops(over):
    assert _call_ex(**over) == 0


SPLIT_GOOD = dict(q=A, k=A, v=A, batch=1, n_heads=2, n_kv_heads=1, ql=8, kl=1000, head_dim=64,
                  scale=0.125, causal=1, n_split=4, workspace=A, workspace_bytes=1 << 20, O=A, L=A,
                  stream=0)


def _call_split(**over):
    args = dict(SPLIT_GOOD)
    args.update(over)
    return fa.fa_train_fwd_split(**args)


def test_split_workspace_size():
    # partial O (f32, 256-byte aligned) then partial L (f32) for every chunk
    rows, D, n = 2 * 4 * 100, 128, 7
    o_bytes = (n * rows * D * 4 + 255) // 256 * 256
    assert fa.fa_train_fwd_split_workspace(2, 4, 100, D, n) == o_bytes + n * rows * 4
    assert fa.fa_train_fwd_split_workspace(2, 4, 100, D, 0) == 0
    assert fa.fa_train_fwd_split_workspace(-1, 4, 100, D, 2) == 0


@pytest.mark.parametrize("over,code", [
    (dict(n_split=0), 11), (dict(n_split=65537), 11), (dict(workspace_bytes=1000), 11),
    (dict(workspace=0), 1), (dict(workspace=A + 8), 6), (dict(q=0), 1), (dict(head_dim=96), 4),
    (dict(n_heads=3, n_kv_heads=2), 3), (dict(scale=math.nan), 5), (dict(kl=-1), 2),
])
def test_split_invalid_arguments_are_rejected(over, code):
    assert _call_split(**over) == code


@pytest.mark.parametrize("over", [dict(batch=0), dict(ql=0, workspace=0)])
def test_split_empty_problems_are_noops(over):
    assert _call_split(**over) == 0


def test_python_binding_fails_loudly_without_gpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.train_fwd(q, q, q)
    with pytest.raises(TypeError):
        fa.train_fwd(q.float(), q, q)
    with pytest.raises(ValueError):
        fa.train_fwd_swa(q, q, q, 4)
    with pytest.raises(ValueError):
        fa.train_fwd_ex(q, q, q, mask=torch.zeros(1, 1, 4, 4, dtype=torch.bfloat16))


BWD_GOOD = dict(q=A, k=A, v=A, mask=0, O=A, L=A, dO=A, batch=1, n_heads=2, n_kv_heads=1, ql=8,
                kl=8, head_dim=64, scale=0.125, causal=0, dQ=A, dK=A, dV=A, stream=0)


def _call_bwd(**over):
    args = dict(BWD_GOOD)
    args.update(over)
    return fa.fa_train_bwd(**args)


@pytest.mark.parametrize("over,code", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(O=0), 1), (dict(L=0), 1),
    (dict(dO=0), 1), (dict(dQ=0), 1), (dict(dK=0), 1), (dict(dV=0), 1),
    (dict(batch=-1), 2), (dict(ql=-1), 2), (dict(kl=-3), 2), (dict(n_heads=0), 2),
    (dict(n_kv_heads=0), 2), (dict(n_heads=3, n_kv_heads=2), 3), (dict(head_dim=96), 4),
    (dict(scale=math.nan), 5), (dict(scale=-math.inf), 5), (dict(q=A + 2), 6),
    (dict(dO=A + 8), 6), (dict(dK=A + 4), 6), (dict(dV=A + 2), 6), (dict(mask=A + 2), 6),
    (dict(L=A + 1), 6), (dict(batch=65536, n_heads=65536, n_kv_heads=1, ql=1), 7),
])
def test_backward_invalid_arguments_are_rejected(over, code):
    assert _call_bwd(**over) == code


@pytest.mark.parametrize("over", [dict(batch=0), dict(ql=0, kl=0),
                                  dict(batch=0, q=0, k=0, v=0, O=0, L=0, dO=0, dQ=0, dK=0, dV=0)])
def test_backward_empty_problems_are_noops(over):
    assert _call_bwd(**over) == 0


def test_backward_window_rejects_negative_window():
    args = {k: v for k, v in BWD_GOOD.items() if k != "causal"}
    assert fa.fa_train_bwd_swa(**args, window=-1) == 9
    assert fa.fa_train_bwd_swa(**dict(args, q=0), window=3) == 1
    assert fa.fa_train_bwd_swa(**dict(args, batch=0), window=3) == 0


def test_backward_binding_fails_loudly_without_gpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    L = torch.zeros(1, 1, 4)
    with pytest.raises(ValueError):
        fa.train_bwd(q, q, q, q, L, q)
    with pytest.raises(TypeError):
        fa.train_bwd(q.float(), q, q, q, L, q)


def test_suggest_n_split():
    assert fa.suggest_n_split(1, 32, 512, 128) == 8     # 64 plain workgroups
    # decoding (at most 16 packed rows, head_dim 64 or 128): one workgroup per
    # CU, at least 8 chunks
    assert fa.suggest_n_split(1, 32, 1, 128) == 8       # 32 plain workgroups
    assert fa.suggest_n_split(8, 32, 1, 128) == 8       # 256: still split
    assert fa.suggest_n_split(8, 32, 1, 128, n_kv_heads=8) == 8   # packed: 64
    assert fa.suggest_n_split(1, 32, 1, 128, n_kv_heads=8) == 32  # packed: 8
    assert fa.suggest_n_split(1, 2, 16, 64) == 128      # 16 rows of 2 heads
    assert fa.suggest_n_split(1, 2, 17, 64) == 256      # 17 rows: two per CU
    assert fa.suggest_n_split(1, 32, 1, 256) == 16      # head_dim 256: two per CU
    assert fa.suggest_n_split(2, 16, 8192, 256) == 1


PAGED_GOOD = dict(q=A, k_cache=A, v_cache=A, block_table=A, seq_lens=A, batch=2, n_heads=4,
                  n_kv_heads=2, ql=1, n_blocks=8, block_size=64, max_blocks=4, head_dim=128,
                  scale=0.1, causal=1, sinks=0, n_split=0, workspace=0, workspace_bytes=0, O=A,
                  L=A, stream=0)


def _call_paged(**over):
    args = dict(PAGED_GOOD)
    args.update(over)
    return fa.fa_paged_fwd(**args)


@pytest.mark.parametrize("over,code", [
    (dict(block_size=8), 12), (dict(block_size=40), 12), (dict(block_size=0), 12),
    (dict(n_blocks=0), 12), (dict(block_table=0), 1), (dict(seq_lens=0), 1), (dict(k_cache=0), 1),
    (dict(q=A + 2), 6), (dict(block_table=A + 2), 6), (dict(seq_lens=A + 1), 6),
    (dict(head_dim=80), 4), (dict(n_heads=3), 3), (dict(scale=math.inf), 5),
    (dict(max_blocks=-1), 2), (dict(n_blocks=-1), 2), (dict(n_split=-1), 11),
    (dict(n_split=4), 1), (dict(n_split=4, workspace=A, workspace_bytes=16), 11),
    (dict(max_blocks=1 << 25, block_size=128), 7), (dict(sinks=A + 2), 6),
])
def test_paged_invalid_arguments_are_rejected(over, code):
    assert _call_paged(**over) == code


@pytest.mark.parametrize("over", [dict(batch=0), dict(ql=0, q=0, O=0, L=0)])
def test_paged_empty_problems_are_noops(over):
    assert _call_paged(**over) == 0


BWD_EX_GOOD = dict({k: v for k, v in BWD_GOOD.items() if k != "mask"}, mask=A, mask_dtype=0,
                   mask_stride_b=0, mask_stride_h=64, window=-1)


@pytest.mark.parametrize("over,code", [
    (dict(mask_dtype=3), 10), (dict(mask_stride_h=-1), 10), (dict(causal=0, window=2), 9),
    (dict(mask=A + 2), 6), (dict(mask=A + 1, mask_dtype=1), 6), (dict(dQ=0), 1),
    (dict(head_dim=96), 4), (dict(scale=math.nan), 5),
])
def test_backward_ex_invalid_arguments_are_rejected(over, code):
    args = dict(BWD_EX_GOOD)
    args.update(over)
    assert fa.fa_train_bwd_ex(**args) == code


STRIDED_GOOD = dict(q=A, q_strides=None, k=A, k_strides=None, v=A, v_strides=None, mask=0,
                    mask_dtype=0, mask_strides=None, batch=1,
                    n_heads=4, n_kv_heads=2, ql=8, kl=8, head_dim=64, scale=0.125, causal=1,
                    window=-1, n_split=0, workspace=0, workspace_bytes=0, O=A, o_strides=None,
                    L=A, stream=0)


@pytest.mark.parametrize("over,code", [
    (dict(q_strides=(-8, 512, 64)), 13), (dict(o_strides=(0, 0, -64)), 13),
    (dict(k_strides=(4096, 64, 12)), 6), (dict(v_strides=(4, 512, 64)), 6),
    (dict(k_strides=(0, 0, 1 << 25)), 7), (dict(n_split=2, window=3), 9),
    (dict(causal=0, window=3), 9), (dict(n_split=-1), 11), (dict(head_dim=72), 4),
    (dict(n_split=2, head_dim=80, workspace=A, workspace_bytes=1 << 20), 4),
    (dict(q=0), 1), (dict(n_split=2), 1), (dict(mask=A, mask_strides=(0, 0, -8)), 10),
    (dict(mask=A, mask_strides=(-1, 0, 8)), 10), (dict(mask=A, n_split=2, workspace=A,
                                                       workspace_bytes=1 << 20), 10),
    (dict(mask=A, mask_dtype=5), 10), (dict(mask=A + 2), 6),
])
def test_strided_invalid_arguments_are_rejected(over, code):
    args = dict(STRIDED_GOOD)
    args.update(over)
    assert fa.fa_train_fwd_strided(**args) == code


DV_GOOD = dict(STRIDED_GOOD, head_dim=96, head_dim_v=64, sinks=0)


@pytest.mark.parametrize("over,code", [
    # (key, value) head dims without kernels
    (dict(head_dim=64, head_dim_v=128), 4), (dict(head_dim=96, head_dim_v=80), 4),
    (dict(head_dim=80, head_dim_v=64), 4), (dict(head_dim=72, head_dim_v=72), 4),
    (dict(head_dim=192, head_dim_v=64), 4), (dict(head_dim=128, head_dim_v=0), 4),
    (dict(q=0), 1), (dict(v=0), 1), (dict(L=0), 1), (dict(kl=-1), 2),
    (dict(n_heads=3, n_kv_heads=2), 3), (dict(scale=math.nan), 5), (dict(v=A + 8), 6),
    (dict(v_strides=(4096, 64, 12)), 6), (dict(o_strides=(0, 0, -64)), 13),
    (dict(causal=0, window=3), 9), (dict(mask=A, mask_dtype=5), 10),
    # O's rows (64 elements) overlap at a row stride of 32
    (dict(o_strides=(4 * 8 * 32, 8 * 32, 32)), 13),
    # sinks: f32, 4-byte aligned; checked like the other operands
    (dict(sinks=A + 2), 6), (dict(sinks=A + 2, head_dim=64, head_dim_v=128), 4),
    # split-KV: equal base widths only, no mask or window, a large enough workspace
    (dict(n_split=2, workspace=A, workspace_bytes=1 << 20), 4),
    (dict(n_split=2, head_dim=80, head_dim_v=80, workspace=A, workspace_bytes=1 << 20), 4),
    (dict(n_split=-1, head_dim=64, head_dim_v=64), 11),
    (dict(n_split=2, head_dim=64, head_dim_v=64, sinks=A, workspace=A, workspace_bytes=16), 11),
    (dict(n_split=2, head_dim=64, head_dim_v=64, window=3), 9),
    (dict(n_split=2, head_dim=64, head_dim_v=64, mask=A), 10),
    (dict(n_split=2, head_dim=64, head_dim_v=64, sinks=A + 2, workspace=A,
          workspace_bytes=1 << 20), 6),
])
def test_dv_invalid_arguments_are_rejected(over, code):
    args = dict(DV_GOOD)
    args.update(over)
    assert fa.fa_train_fwd_dv(**args) == code


@pytest.mark.parametrize("over", [dict(batch=0), dict(ql=0, q=0, k=0, v=0, O=0, L=0),
                                  dict(batch=0, sinks=A)])
def test_dv_empty_problems_are_noops(over):
    args = dict(DV_GOOD)
    args.update(over)
    assert fa.fa_train_fwd_dv(**args) == 0


def test_base_dims_only_where_stated():
    # split-KV, paged, no-alloc and backward keep to 64, 128 and 256
    sp = dict(SPLIT_GOOD, head_dim=80)
    assert fa.fa_train_fwd_split(**sp) == 4
    assert fa.fa_train_fwd_split(**dict(SPLIT_GOOD, head_dim=192)) == 4
    assert "80, 96" in fa.status_string(4)


def test_strided_status_string():
    assert "stride" in fa.status_string(13)


BWD_STRIDED_GOOD = dict(q=A, k=A, v=A, O=A, L=A, dO=A, q_strides=None, kv_strides=None, mask=0,
                        mask_dtype=0, mask_strides=None, batch=1,
                        n_heads=4, n_kv_heads=2, ql=8, kl=8, head_dim=64, scale=0.125, causal=1,
                        window=-1, dQ=A, dK=A, dV=A, stream=0)


@pytest.mark.parametrize("over,code", [
    (dict(q_strides=(-8, 512, 64)), 13), (dict(kv_strides=(0, 0, -64)), 13),
    (dict(kv_strides=(4096, 64, 12)), 6), (dict(q_strides=(4, 512, 64)), 6),
    (dict(q_strides=(0, 0, 1 << 25)), 7), (dict(causal=0, window=3), 9), (dict(head_dim=96), 4),
    (dict(dQ=0), 1), (dict(mask=A, mask_strides=(0, 0, -8)), 10), (dict(mask=A, mask_dtype=3), 10),
])
def test_bwd_strided_invalid_arguments_are_rejected(over, code):
    args = dict(BWD_STRIDED_GOOD)
    args.update(over)
    assert fa.fa_train_bwd_strided(**args) == code


BWD_SINKS_GOOD = dict(BWD_STRIDED_GOOD, sinks=A, dsinks=A)


@pytest.mark.parametrize("over,code", [
    (dict(dsinks=0), 1), (dict(sinks=A + 2), 6), (dict(dsinks=A + 2), 6), (dict(dQ=0), 1),
    (dict(head_dim=96), 4), (dict(q_strides=(-8, 512, 64)), 13), (dict(causal=0, window=3), 9),
])
def test_bwd_sinks_invalid_arguments_are_rejected(over, code):
    """Host checks of fa_train_bwd_sinks, before any HIP call (no GPU here)."""
    args = dict(BWD_SINKS_GOOD)
    args.update(over)
    assert fa.fa_train_bwd_sinks(**args) == code


def test_bwd_sinks_binding_fails_loudly_without_gpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    L = torch.zeros(1, 1, 4)
    with pytest.raises(ValueError):
        fa.train_bwd_sinks(q, q, q, q, L, q, torch.zeros(1))


def test_strided_and_paged_bindings_fail_loudly_without_gpu_tensors():
    """No CPU path: CPU tensors are refused before any library call."""
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    L = torch.zeros(1, 1, 4)
    with pytest.raises(ValueError):
        fa.train_fwd_strided(q, q, q)
    with pytest.raises(ValueError):
        fa.train_fwd_strided(q.transpose(1, 2), q, q)
    with pytest.raises(ValueError):
        fa.train_bwd_strided(q, q, q, q, L, q)
    with pytest.raises(ValueError):
        fa.train_bwd_ex(q, q, q, q, L, q)
    with pytest.raises(ValueError):
        fa.train_fwd_split(q, q, q, 2)


NOALLOC_GOOD = dict(q=A, k=A, v=A, batch=1, n_heads=2, n_kv_heads=1, ql=8, kl=1000, head_dim=64,
                    scale=0.125, causal=1, n_split=4, O=A, L=A, stream=0)


@pytest.mark.parametrize("over,code", [
    (dict(n_split=0), 11), (dict(n_split=65537), 11), (dict(batch=-1), 2), (dict(n_heads=0), 2),
    (dict(head_dim=96), 4),
    # partials above the 16 MiB scratch: 4 * 32 * 512 rows * 128 dims * 4 B * 8 chunks
    (dict(batch=4, n_heads=32, n_kv_heads=8, ql=512, kl=4096, head_dim=128, n_split=8), 14),
])
def test_noalloc_invalid_arguments_are_rejected(over, code):
    """Checked on the host before the scratch is located or anything runs."""
    args = dict(NOALLOC_GOOD)
    args.update(over)
    assert fa.fa_train_fwd_split_noalloc(**args) == code


@pytest.mark.parametrize("over", [dict(batch=0), dict(ql=0, q=0, O=0, L=0)])
def test_noalloc_empty_problems_are_noops(over):
    args = dict(NOALLOC_GOOD)
    args.update(over)
    assert fa.fa_train_fwd_split_noalloc(**args) == 0


def test_noalloc_scratch_size_matches_header():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    assert "#define FA_NOALLOC_SCRATCH_BYTES (16ul << 20)" in text
    assert fa.NOALLOC_SCRATCH_BYTES == 16 << 20
