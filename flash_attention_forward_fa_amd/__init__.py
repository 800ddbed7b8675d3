"""Flash-attention training forward (O and L) and backward (dQ, dK, dV) on AMD
MI355X.

A thin binding over libfa.so (include/fa.h): argument marshalling only. Every
step of the computation runs in the library's gfx950 kernels; PyTorch only
provides device memory and the current stream. There is no fallback: if the
library is missing or the tensors are not on a GPU, the call raises.
"""
import ctypes
import math
import os

from . import build as _build

LIB_PATH = _build.LIB

FA_STATUS = {
    0: "FA_OK", 1: "FA_ERR_NULL_POINTER", 2: "FA_ERR_BAD_SIZE", 3: "FA_ERR_HEAD_GROUPING",
    4: "FA_ERR_HEAD_DIM", 5: "FA_ERR_SCALE", 6: "FA_ERR_ALIGNMENT", 7: "FA_ERR_TOO_LARGE",
    8: "FA_ERR_LAUNCH", 9: "FA_ERR_WINDOW", 10: "FA_ERR_MASK", 11: "FA_ERR_SPLIT",
    12: "FA_ERR_PAGED",
    13: "FA_ERR_STRIDE", 14: "FA_ERR_SCRATCH",
}
# Bytes of the library-held scratch of fa_train_fwd_split_noalloc (per GPU).
NOALLOC_SCRATCH_BYTES = 16 << 20
FA_MASK_F32, FA_MASK_BF16, FA_MASK_BOOL = 0, 1, 2

_lib = None


class FAError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{FA_STATUS.get(status, status)}: {message}")
        self.status = status


def lib():
    """The loaded C library (ctypes). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m flash_attention_forward_fa_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        vp, ci = ctypes.c_void_p, ctypes.c_int
        l.fa_train_fwd.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ctypes.c_float, ci,
                                   vp, vp, vp]
        l.fa_train_fwd.restype = ci
        l.fa_train_fwd_swa.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ctypes.c_float,
                                       ci, vp, vp, vp]
        l.fa_train_fwd_swa.restype = ci
        i64 = ctypes.c_longlong
        l.fa_train_fwd_ex.argtypes = [vp, vp, vp, vp, ci, i64, i64, ci, ci, ci, ci, ci, ci,
                                      ctypes.c_float, ci, ci, vp, vp, vp]
        l.fa_train_fwd_ex.restype = ci
        pll = ctypes.POINTER(ctypes.c_longlong)
        l.fa_train_fwd_strided.argtypes = [vp, pll, vp, pll, vp, pll, vp, ci, pll, ci, ci, ci, ci,
                                           ci, ci,
                                           ctypes.c_float, ci, ci, ci, vp, ctypes.c_ulong, vp,
                                           pll, vp, vp]
        l.fa_train_fwd_strided.restype = ci
        l.fa_train_fwd_dv.argtypes = [vp, pll, vp, pll, vp, pll, vp, ci, pll, ci, ci, ci, ci, ci,
                                      ci, ci, ctypes.c_float, ci, ci, vp, ci, vp, ctypes.c_ulong,
                                      vp, pll, vp, vp]
        l.fa_train_fwd_dv.restype = ci
        l.fa_train_bwd_strided.argtypes = [vp, vp, vp, vp, vp, vp, pll, pll, vp, ci, pll, ci, ci,
                                           ci, ci, ci, ci, ctypes.c_float, ci, ci, vp, vp, vp, vp]
        l.fa_train_bwd_strided.restype = ci
        l.fa_train_bwd_sinks.argtypes = [vp, vp, vp, vp, vp, vp, pll, pll, vp, ci, pll, ci, ci,
                                         ci, ci, ci, ci, ctypes.c_float, ci, ci, vp, vp, vp, vp,
                                         vp, vp]
        l.fa_train_bwd_sinks.restype = ci
        ul = ctypes.c_ulong
        l.fa_train_fwd_split.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ci, ctypes.c_float, ci,
                                         ci, vp, ul, vp, vp, vp]
        l.fa_train_fwd_split.restype = ci
        l.fa_train_fwd_split_noalloc.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ci,
                                                 ctypes.c_float, ci, ci, vp, vp, vp]
        l.fa_train_fwd_split_noalloc.restype = ci
        l.fa_train_fwd_split_workspace.argtypes = [ci, ci, ci, ci, ci]
        l.fa_train_fwd_split_workspace.restype = ul
        l.fa_paged_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci,
                                   ctypes.c_float, ci, vp, ci, vp, ul, vp, vp, vp]
        l.fa_paged_fwd.restype = ci
        l.fa_train_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci,
                                   ctypes.c_float, ci, vp, vp, vp, vp]
        l.fa_train_bwd.restype = ci
        l.fa_train_bwd_swa.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci,
                                       ctypes.c_float, ci, vp, vp, vp, vp]
        l.fa_train_bwd_swa.restype = ci
        l.fa_train_bwd_ex.argtypes = [vp, vp, vp, vp, ci, ctypes.c_longlong, ctypes.c_longlong,
                                      vp, vp, vp, ci, ci, ci, ci, ci, ci, ctypes.c_float, ci, ci,
                                      vp, vp, vp, vp]
        l.fa_train_bwd_ex.restype = ci
        l.fa_status_string.argtypes = [ci]
        l.fa_status_string.restype = ctypes.c_char_p
        _lib = l
    return _lib


def status_string(status):
    return lib().fa_status_string(int(status)).decode()


def _on_gpu(t):
    """Whether tensor t lives in GPU memory (the kernels take device pointers only)."""
    return t.is_cuda


def _check_out(t, name, dev, dtype, shape, layout="contiguous"):
    """Checks a caller-supplied output (or workspace) tensor before its pointer
    reaches the library: a torch tensor of `dtype` and exactly `shape` on the
    GPU `dev` (q's device), with layout "contiguous" or "rows" (only the last
    dimension must be contiguous; the library then checks the strides)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not _on_gpu(t) or t.device != dev:
        raise ValueError(f"{name} must be on {dev}, got {t.device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if layout == "contiguous" and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if layout == "rows" and t.dim() and t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have a contiguous last dimension")
    return t


def _check_workspace(ws, need, dev):
    """A split-KV workspace: a contiguous uint8 tensor on `dev` of at least
    `need` bytes."""
    import torch
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 torch tensor")
    if not _on_gpu(ws) or ws.device != dev:
        raise ValueError(f"workspace must be on {dev}, got {ws.device}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, the call needs {need}")
    return ws


def _check_inputs(tensors, dev, layout="contiguous"):
    """q, k, v (and O, dO) inputs: bf16 4-d tensors on the GPU `dev`."""
    import torch
    for name, t in tensors:
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be a bfloat16 tensor")
        if t.dim() != 4 or not _on_gpu(t) or t.device != dev:
            raise ValueError(f"{name} must be a 4-d tensor on {dev}")
        if layout == "contiguous" and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if layout == "rows" and t.shape[-1] > 1 and t.stride(3) != 1:
            raise ValueError(f"{name} must have a contiguous head_dim")


def _non_overlapping(shape, strides):
    """Whether no two elements of a view share an address: the dimensions of
    size > 1, sorted by stride, each step at least the span of those below."""
    dims = sorted((st, n) for n, st in zip(shape, strides) if n > 1)
    span = 1
    for st, n in dims:
        if st < span:
            return False
        span = st * (n - 1) + span
    return True


def fa_train_fwd(q, k, v, mask, batch, n_heads, n_kv_heads, ql, kl, head_dim, scale, causal,
                 O, L, stream):
    """The C entry point with raw integer pointers (0 for NULL); returns the status."""
    return lib().fa_train_fwd(q or None, k or None, v or None, mask or None, batch, n_heads,
                              n_kv_heads, ql, kl, head_dim, float(scale), int(bool(causal)),
                              O or None, L or None, stream or None)


def fa_train_fwd_swa(q, k, v, mask, batch, n_heads, n_kv_heads, ql, kl, head_dim, scale, window,
                     O, L, stream):
    """The C entry point with raw integer pointers (0 for NULL); returns the status."""
    return lib().fa_train_fwd_swa(q or None, k or None, v or None, mask or None, batch, n_heads,
                                  n_kv_heads, ql, kl, head_dim, float(scale), int(window),
                                  O or None, L or None, stream or None)


def fa_train_fwd_ex(q, k, v, mask, mask_dtype, mask_stride_b, mask_stride_h, batch, n_heads,
                    n_kv_heads, ql, kl, head_dim, scale, causal, window, O, L, stream):
    """The C entry point with raw integer pointers (0 for NULL); returns the status."""
    return lib().fa_train_fwd_ex(q or None, k or None, v or None, mask or None, int(mask_dtype),
                                 int(mask_stride_b), int(mask_stride_h), batch, n_heads,
                                 n_kv_heads, ql, kl, head_dim, float(scale), int(bool(causal)),
                                 int(window), O or None, L or None, stream or None)


def train_fwd_ex(q, k, v, mask=None, scale=None, causal=False, window=None, out=None, lse=None,
                 stream=None):
    """O, L = train_fwd_ex(q, k, v, mask=None, scale=None, causal=False, window=None)

    train_fwd with every option of fa_train_fwd_ex: mask may be float32 or
    bfloat16 (additive) or bool (True = visible), of shape [B or 1, H or 1, ql,
    kl] (a size-1 batch or head dim is broadcast; any batch/head strides, rows
    contiguous); window (>= 0, with causal=True) selects the sliding window of
    train_fwd_swa.
    """
    import torch

    if mask is None:
        return _train_fwd(q, k, v, None, scale, causal, window, out, lse, stream, ex=True)
    if mask.dtype not in (torch.float32, torch.bfloat16, torch.bool):
        raise ValueError("mask must be float32, bfloat16 or bool")
    B, H, ql, _ = q.shape
    kl = k.shape[2]
    if (mask.dim() != 4 or mask.shape[0] not in (1, B) or mask.shape[1] not in (1, H)
            or tuple(mask.shape[2:]) != (ql, kl)):
        raise ValueError(f"mask must have shape [B or 1, H or 1, {ql}, {kl}]")
    if ql * kl > 0 and ((kl > 1 and mask.stride(3) != 1) or (ql > 1 and mask.stride(2) != kl)):
        raise ValueError("mask rows must be contiguous (strides [.., .., kl, 1])")
    sb = mask.stride(0) if mask.shape[0] > 1 else 0
    sh = mask.stride(1) if mask.shape[1] > 1 else 0
    return _train_fwd(q, k, v, mask, scale, causal, window, out, lse, stream, ex=True,
                      mask_layout=({torch.bfloat16: FA_MASK_BF16, torch.bool: FA_MASK_BOOL}
                                   .get(mask.dtype, FA_MASK_F32), sb, sh))


def fa_train_fwd_split(q, k, v, batch, n_heads, n_kv_heads, ql, kl, head_dim, scale, causal,
                       n_split, workspace, workspace_bytes, O, L, stream):
    """The C entry point with raw integer pointers (0 for NULL); returns the status."""
    return lib().fa_train_fwd_split(q or None, k or None, v or None, batch, n_heads, n_kv_heads,
                                    ql, kl, head_dim, float(scale), int(bool(causal)),
                                    int(n_split), workspace or None, int(workspace_bytes),
                                    O or None, L or None, stream or None)


def suggest_n_split(batch, n_heads, ql, head_dim, n_kv_heads=None, n_cu=256):
    """Chunks for train_fwd_split: about two workgroups per CU in total, or 1
    (use train_fwd) when the plain launch already has one per CU. With one
    query row per head and GQA (no mask, no window) the library runs a kv
    group's query heads as one packed head: batch * n_kv_heads launch rows.
    At most 16 (packed) query rows with head_dim 64 or 128 (decoding) run the
    library's key-split decode kernel, which beats the plain launch at any
    batch: about one workgroup per CU, and at least 8 chunks (measured best
    on MI355X for batch 1, 4 and 8 against 32k keys)."""
    rows = 128 if head_dim == 256 else 256
    if ql == 1 and n_kv_heads and n_heads > n_kv_heads:
        n_heads, ql = n_kv_heads, n_heads // n_kv_heads
    plain = batch * n_heads * ((ql + rows - 1) // rows)
    if ql <= 16 and head_dim in (64, 128):
        return max(8, (n_cu + plain - 1) // plain)
    return 1 if plain >= n_cu else max(1, (2 * n_cu + plain - 1) // plain)


def fa_train_fwd_split_noalloc(q, k, v, batch, n_heads, n_kv_heads, ql, kl, head_dim, scale,
                               causal, n_split, O, L, stream):
    """The C entry point with raw integer pointers (0 for NULL); returns the status."""
    return lib().fa_train_fwd_split_noalloc(q or None, k or None, v or None, batch, n_heads,
                                            n_kv_heads, ql, kl, head_dim, float(scale),
                                            int(bool(causal)), int(n_split), O or None,
                                            L or None, stream or None)


def train_fwd_split_noalloc(q, k, v, n_split, scale=None, causal=False, out=None, lse=None,
                            stream=None):
    """O, L = train_fwd_split_noalloc(q, k, v, n_split, scale=None, causal=False)

    train_fwd_split with the partials in the library's own per-GPU scratch
    (NOALLOC_SCRATCH_BYTES) instead of a workspace: the library allocates
    nothing (pass out and lse to allocate nothing here either). Calls that may
    overlap on one GPU share that scratch and must be ordered by the caller.
    """
    O, L, (B, H, Hkv, ql, kl, D), scale, s = _fwd_outputs(q, k, v, scale, out, lse, stream)
    import torch
    with torch.cuda.device(q.device):
        status = fa_train_fwd_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, Hkv,
                                            ql, kl, D, scale, causal, n_split, O.data_ptr(),
                                            L.data_ptr(), s.cuda_stream)
    if status != 0:
        raise FAError(status, status_string(status))
    return O, L


def fa_train_fwd_split_workspace(batch, n_heads, ql, head_dim, n_split):
    """Workspace bytes fa_train_fwd_split needs (0 for invalid sizes)."""
    return int(lib().fa_train_fwd_split_workspace(batch, n_heads, ql, head_dim, n_split))


def train_fwd_split(q, k, v, n_split, scale=None, causal=False, workspace=None, out=None,
                    lse=None, stream=None):
    """O, L = train_fwd_split(q, k, v, n_split, scale=None, causal=False, workspace=None)

    train_fwd (no mask) with the keys split into up to n_split chunks computed
    by separate workgroups and merged through their logsumexps: for few query
    tiles against many keys. workspace: a uint8 device tensor of at least
    fa_train_fwd_split_workspace(...) bytes (allocated here when None).
    """
    import torch

    O, L, (B, H, Hkv, ql, kl, D), scale, s = _fwd_outputs(q, k, v, scale, out, lse, stream)
    # (no keys: the library reads no workspace)
    need = fa_train_fwd_split_workspace(B, H, ql, D, n_split) if kl > 0 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, need, q.device)
    with torch.cuda.device(q.device):
        status = fa_train_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, Hkv, ql, kl,
                                    D, scale, causal, n_split, workspace.data_ptr(),
                                    workspace.numel(), O.data_ptr(), L.data_ptr(), s.cuda_stream)
    if status != 0:
        raise FAError(status, status_string(status))
    return O, L


def fa_paged_fwd(q, k_cache, v_cache, block_table, seq_lens, batch, n_heads, n_kv_heads, ql,
                 n_blocks, block_size, max_blocks, head_dim, scale, causal, sinks, n_split,
                 workspace, workspace_bytes, O, L, stream):
    """The C entry point with raw integer pointers (0 for NULL); returns the status."""
    return lib().fa_paged_fwd(q or None, k_cache or None, v_cache or None, block_table or None,
                              seq_lens or None, batch, n_heads, n_kv_heads, ql, n_blocks,
                              block_size, max_blocks, head_dim, float(scale), int(bool(causal)),
                              sinks or None, int(n_split), workspace or None,
                              int(workspace_bytes), O or None, L or None, stream or None)


def paged_fwd(q, k_cache, v_cache, block_table, seq_lens, scale=None, causal=False, n_split=0,
              workspace=None, sinks=None, out=None, lse=None, stream=None):
    """O, L = paged_fwd(q, k_cache, v_cache, block_table, seq_lens, scale=None, causal=False,
                        n_split=0, workspace=None, sinks=None)

    q: bf16 [B, H, ql, D]; k_cache, v_cache: bf16 [n_blocks, Hkv, block_size, D]
    (block_size a positive multiple of 16);
    block_table: int32 [B, max_blocks]; seq_lens: int32 [B] (all on q's GPU).
    Sequence b attends to its first seq_lens[b] keys (key position p at row
    p % block_size of block block_table[b, p // block_size]). n_split > 0 uses
    split-KV with a workspace (allocated here when None). sinks: None or a
    float32 tensor [H] on q's device, as for train_fwd_dv.
    """
    import torch

    if not isinstance(q, torch.Tensor):
        raise TypeError("q must be a bfloat16 tensor")
    _check_inputs((("q", q), ("k_cache", k_cache), ("v_cache", v_cache)), q.device)
    for name, t in (("block_table", block_table), ("seq_lens", seq_lens)):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or not t.is_contiguous()
                or not _on_gpu(t) or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous int32 tensor on q's device")
    B, H, ql, D = q.shape
    n_blocks, Hkv, bs, Dk = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape) or Dk != D:
        raise ValueError("k_cache and v_cache must be [n_blocks, Hkv, block_size, D]")
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table must be [B, max_blocks] and seq_lens [B]")
    max_blocks = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    O = out if out is not None else torch.empty_like(q)
    L = lse if lse is not None else torch.empty((B, H, ql), dtype=torch.float32, device=q.device)
    _check_out(O, "out", q.device, torch.bfloat16, (B, H, ql, D))
    _check_out(L, "lse", q.device, torch.float32, (B, H, ql))
    if sinks is not None:
        _check_out(sinks, "sinks", q.device, torch.float32, (H,))
    ws_ptr, ws_bytes = 0, 0
    if n_split > 0:
        # (a table that addresses no keys needs no workspace)
        need = fa_train_fwd_split_workspace(B, H, ql, D, n_split) if max_blocks * bs > 0 else 0
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        _check_workspace(workspace, need, q.device)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        status = fa_paged_fwd(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                              block_table.data_ptr(), seq_lens.data_ptr(), B, H, Hkv, ql,
                              n_blocks, bs, max_blocks, D, scale, causal,
                              sinks.data_ptr() if sinks is not None else 0, n_split, ws_ptr,
                              ws_bytes, O.data_ptr(), L.data_ptr(), s.cuda_stream)
    if status != 0:
        raise FAError(status, status_string(status))
    return O, L


def _strides3(st):
    """A (batch, head, row) element-stride triple as a C array, or None."""
    if st is None:
        return None
    return (ctypes.c_longlong * 3)(*(int(x) for x in st))


def fa_train_fwd_strided(q, q_strides, k, k_strides, v, v_strides, mask, mask_dtype,
                         mask_strides, batch, n_heads, n_kv_heads, ql, kl, head_dim, scale, causal,
                         window, n_split, workspace, workspace_bytes, O, o_strides, L, stream):
    """The C entry point with raw integer pointers (0 for NULL) and stride
    triples (or None); returns the status."""
    return lib().fa_train_fwd_strided(
        q or None, _strides3(q_strides), k or None, _strides3(k_strides), v or None,
        _strides3(v_strides), mask or None, int(mask_dtype), _strides3(mask_strides), batch,
        n_heads, n_kv_heads, ql, kl, head_dim, float(scale),
        int(bool(causal)), int(window), int(n_split), workspace or None, int(workspace_bytes),
        O or None, _strides3(o_strides), L or None, stream or None)


def _mask_view(mask, q, k):
    """(pointer, dtype code, strides) of a mask view [B or 1, H or 1, ql, kl]
    with contiguous keys (any row stride), or (0, 0, None) for none."""
    import torch
    if mask is None:
        return 0, FA_MASK_F32, None
    if not isinstance(mask, torch.Tensor) or mask.dtype not in (torch.float32, torch.bfloat16,
                                                                 torch.bool):
        raise ValueError("mask must be float32, bfloat16 or bool")
    B, H, ql, _ = q.shape
    kl = k.shape[2]
    if (mask.dim() != 4 or mask.shape[0] not in (1, B) or mask.shape[1] not in (1, H)
            or tuple(mask.shape[2:]) != (ql, kl)):
        raise ValueError(f"mask must have shape [B or 1, H or 1, {ql}, {kl}]")
    if kl > 1 and mask.stride(3) != 1:
        raise ValueError("the mask's keys must be contiguous")
    if not _on_gpu(mask) or mask.device != q.device:
        raise ValueError("mask must be on q's device")
    st = (mask.stride(0) if mask.shape[0] > 1 else 0, mask.stride(1) if mask.shape[1] > 1 else 0,
          mask.stride(2) if ql > 1 else kl)
    code = {torch.bfloat16: FA_MASK_BF16, torch.bool: FA_MASK_BOOL}.get(mask.dtype, FA_MASK_F32)
    return mask.data_ptr(), code, st


def train_fwd_strided(q, k, v, mask=None, scale=None, causal=False, window=None, n_split=0,
                      workspace=None, out=None, lse=None, stream=None):
    """O, L = train_fwd_strided(q, k, v, scale=None, causal=False, window=None, n_split=0)

    The forward on strided views: q [B, H, ql, D], k and v [B, Hkv, kl, D] and
    out (optional, else a new contiguous tensor) may have any non-negative
    strides in their first three dimensions (multiples of 8 elements) with
    head_dim contiguous, e.g. q = x.transpose(1, 2) for x of layout
    [B, ql, H, D]. L is contiguous [B, H, ql]. mask: as for train_fwd_ex, any
    view whose keys are contiguous (e.g. a slice [..., :ql, :kl] of a larger
    mask). n_split > 0 runs split-KV (its workspace allocated here when None).
    """
    import torch
    if not isinstance(q, torch.Tensor):
        raise TypeError("q must be a bfloat16 tensor")
    _check_inputs((("q", q), ("k", k), ("v", v)), q.device, layout="rows")
    B, H, ql, D = q.shape
    Bk, Hkv, kl, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError("k and v must be [B, Hkv, kl, D] with q's B and D")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    O = out if out is not None else torch.empty((B, H, ql, D), dtype=torch.bfloat16,
                                                device=q.device)
    L = lse if lse is not None else torch.empty((B, H, ql), dtype=torch.float32, device=q.device)
    _check_out(O, "out", q.device, torch.bfloat16, (B, H, ql, D), layout="rows")
    if not _non_overlapping(O.shape, O.stride()):
        raise ValueError("out must not have overlapping rows (its strides alias elements)")
    _check_out(L, "lse", q.device, torch.float32, (B, H, ql))
    ws_bytes = 0
    if n_split > 0:
        ws_bytes = fa_train_fwd_split_workspace(B, H, ql, D, n_split) if kl > 0 else 0
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
        _check_workspace(workspace, ws_bytes, q.device)
        ws_bytes = workspace.numel()
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    st = lambda t: t.stride()[:3]
    mptr, mdt, mst = _mask_view(mask, q, k)
    with torch.cuda.device(q.device):
        status = fa_train_fwd_strided(
            q.data_ptr(), st(q), k.data_ptr(), st(k), v.data_ptr(), st(v), mptr, mdt, mst,
            B, H, Hkv, ql, kl, D,
            scale, causal, -1 if window is None else window, n_split,
            workspace.data_ptr() if workspace is not None else 0, ws_bytes, O.data_ptr(), st(O),
            L.data_ptr(), s.cuda_stream)
    if status != 0:
        raise FAError(status, status_string(status))
    return O, L


def fa_train_fwd_dv(q, q_strides, k, k_strides, v, v_strides, mask, mask_dtype, mask_strides,
                    batch, n_heads, n_kv_heads, ql, kl, head_dim, head_dim_v, scale, causal,
                    window, sinks, n_split, workspace, workspace_bytes, O, o_strides, L, stream):
    """The C entry point with raw integer pointers (0 for NULL) and stride
    triples (or None); returns the status."""
    return lib().fa_train_fwd_dv(
        q or None, _strides3(q_strides), k or None, _strides3(k_strides), v or None,
        _strides3(v_strides), mask or None, int(mask_dtype), _strides3(mask_strides), batch,
        n_heads, n_kv_heads, ql, kl, head_dim, head_dim_v, float(scale), int(bool(causal)),
        int(window), sinks or None, int(n_split), workspace or None, int(workspace_bytes),
        O or None, _strides3(o_strides), L or None, stream or None)


def train_fwd_dv(q, k, v, mask=None, scale=None, causal=False, window=None, sinks=None,
                 n_split=0, workspace=None, out=None, lse=None, stream=None):
    """O, L = train_fwd_dv(q, k, v, mask=None, scale=None, causal=False, window=None,
                           sinks=None, n_split=0)

    The forward with a value head dim Dv that may differ from the key head dim
    D: q [B, H, ql, D], k [B, Hkv, kl, D], v [B, Hkv, kl, Dv], out [B, H, ql, Dv]
    (strided views as for train_fwd_strided), (D, Dv) one of (64, 64),
    (80, 80), (96, 96), (96, 64), (128, 128), (192, 192), (192, 128),
    (256, 256). mask, window, scale (default 1/sqrt(D)) as for
    train_fwd_strided; L is contiguous [B, H, ql]. sinks: None or a float32
    tensor [H] on q's device, one logit per query head that joins every row's
    softmax as one more term with a zero value (include/fa.h). n_split > 0
    runs split-KV (Dv == D in {64, 128, 256}, no mask or window; the
    workspace allocated here when None).
    """
    import torch
    if not isinstance(q, torch.Tensor):
        raise TypeError("q must be a bfloat16 tensor")
    _check_inputs((("q", q), ("k", k), ("v", v)), q.device, layout="rows")
    B, H, ql, D = q.shape
    Bk, Hkv, kl, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape[:3]) != (B, Hkv, kl):
        raise ValueError("k must be [B, Hkv, kl, D] and v [B, Hkv, kl, Dv] with q's B and D")
    Dv = v.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    O = out if out is not None else torch.empty((B, H, ql, Dv), dtype=torch.bfloat16,
                                                device=q.device)
    L = lse if lse is not None else torch.empty((B, H, ql), dtype=torch.float32, device=q.device)
    _check_out(O, "out", q.device, torch.bfloat16, (B, H, ql, Dv), layout="rows")
    if not _non_overlapping(O.shape, O.stride()):
        raise ValueError("out must not have overlapping rows (its strides alias elements)")
    _check_out(L, "lse", q.device, torch.float32, (B, H, ql))
    if sinks is not None:
        _check_out(sinks, "sinks", q.device, torch.float32, (H,))
    ws_bytes = 0
    if n_split > 0:
        ws_bytes = fa_train_fwd_split_workspace(B, H, ql, Dv, n_split) if kl > 0 else 0
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
        _check_workspace(workspace, ws_bytes, q.device)
        ws_bytes = workspace.numel()
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    st = lambda t: t.stride()[:3]
    mptr, mdt, mst = _mask_view(mask, q, k)
    with torch.cuda.device(q.device):
        status = fa_train_fwd_dv(
            q.data_ptr(), st(q), k.data_ptr(), st(k), v.data_ptr(), st(v), mptr, mdt, mst,
            B, H, Hkv, ql, kl, D, Dv, scale, causal, -1 if window is None else window,
            sinks.data_ptr() if sinks is not None else 0, n_split,
            workspace.data_ptr() if workspace is not None else 0, ws_bytes, O.data_ptr(), st(O),
            L.data_ptr(), s.cuda_stream)
    if status != 0:
        raise FAError(status, status_string(status))
    return O, L


def fa_train_bwd_strided(q, k, v, O, L, dO, q_strides, kv_strides, mask, mask_dtype,
                         mask_strides, batch, n_heads, n_kv_heads, ql, kl, head_dim, scale, causal,
                         window, dQ, dK, dV, stream):
    """The C entry point with raw integer pointers (0 for NULL) and stride
    triples (or None); returns the status."""
    return lib().fa_train_bwd_strided(
        q or None, k or None, v or None, O or None, L or None, dO or None, _strides3(q_strides),
        _strides3(kv_strides), mask or None, int(mask_dtype), _strides3(mask_strides), batch, n_heads, n_kv_heads, ql, kl, head_dim, float(scale),
        int(bool(causal)), int(window), dQ or None, dK or None, dV or None, stream or None)


def train_bwd_strided(q, k, v, O, L, dO, mask=None, scale=None, causal=False, window=None,
                      stream=None):
    """dQ, dK, dV = train_bwd_strided(q, k, v, O, L, dO, scale=None, causal=False,
                                      window=None)

    The backward on strided views: O and dO must have q's strides, v k's
    (head_dim contiguous); dQ comes in q's layout, dK and dV in k's.
    """
    import torch
    if not isinstance(q, torch.Tensor):
        raise TypeError("q must be a bfloat16 tensor")
    _check_inputs((("q", q), ("k", k), ("v", v), ("O", O), ("dO", dO)), q.device, layout="rows")
    B, H, ql, D = q.shape
    Bk, Hkv, kl, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError("k and v must be [B, Hkv, kl, D] with q's B and D")
    if O.shape != q.shape or dO.shape != q.shape:
        raise ValueError("O and dO must be shaped like q")
    if O.stride() != q.stride() or dO.stride() != q.stride() or v.stride() != k.stride():
        raise ValueError("O and dO need q's strides, v needs k's")
    _check_out(L, "L", q.device, torch.float32, (B, H, ql))
    # dQ takes q's stride triple and dK, dV take k's: a view whose elements
    # alias (e.g. K expanded over the batch) would make workgroups write the
    # same gradient rows, so such inputs are copied to a contiguous layout first
    if not _non_overlapping(q.shape, q.stride()):
        q, O, dO = q.contiguous(), O.contiguous(), dO.contiguous()
    if not _non_overlapping(k.shape, k.stride()):
        k, v = k.contiguous(), v.contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dQ = torch.empty_strided(q.shape, q.stride(), dtype=torch.bfloat16, device=q.device)
    dK = torch.empty_strided(k.shape, k.stride(), dtype=torch.bfloat16, device=q.device)
    dV = torch.empty_strided(k.shape, k.stride(), dtype=torch.bfloat16, device=q.device)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    mptr, mdt, mst = _mask_view(mask, q, k)
    with torch.cuda.device(q.device):
        status = fa_train_bwd_strided(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), O.data_ptr(), L.data_ptr(), dO.data_ptr(),
            q.stride()[:3], k.stride()[:3], mptr, mdt, mst, B, H, Hkv, ql, kl, D, scale, causal,
            -1 if window is None else window, dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(),
            s.cuda_stream)
    if status != 0:
        raise FAError(status, status_string(status))
    return dQ, dK, dV


def fa_train_bwd_sinks(q, k, v, O, L, dO, q_strides, kv_strides, mask, mask_dtype,
                       mask_strides, batch, n_heads, n_kv_heads, ql, kl, head_dim, scale, causal,
                       window, sinks, dQ, dK, dV, dsinks, stream):
    """The C entry point with raw integer pointers (0 for NULL) and stride
    triples (or None); returns the status."""
    return lib().fa_train_bwd_sinks(
        q or None, k or None, v or None, O or None, L or None, dO or None, _strides3(q_strides),
        _strides3(kv_strides), mask or None, int(mask_dtype), _strides3(mask_strides), batch,
        n_heads, n_kv_heads, ql, kl, head_dim, float(scale), int(bool(causal)), int(window),
        sinks or None, dQ or None, dK or None, dV or None, dsinks or None, stream or None)


def train_bwd_sinks(q, k, v, O, L, dO, sinks, mask=None, scale=None, causal=False, window=None,
                    stream=None):
    """dQ, dK, dV, dsinks = train_bwd_sinks(q, k, v, O, L, dO, sinks, mask=None,
                                          scale=None, causal=False, window=None)

    The backward of train_fwd_dv with sinks (float32 [H] on q's device; the
    value width equal to the key width): the gradients of train_bwd_strided
    (O and L from that forward, with the same sinks), and dsinks, float32 [H],
    the gradient of each query head's sink logit.
    """
    import torch
    if not isinstance(q, torch.Tensor):
        raise TypeError("q must be a bfloat16 tensor")
    _check_inputs((("q", q), ("k", k), ("v", v), ("O", O), ("dO", dO)), q.device, layout="rows")
    B, H, ql, D = q.shape
    Bk, Hkv, kl, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError("k and v must be [B, Hkv, kl, D] with q's B and D")
    if O.shape != q.shape or dO.shape != q.shape:
        raise ValueError("O and dO must be shaped like q")
    if O.stride() != q.stride() or dO.stride() != q.stride() or v.stride() != k.stride():
        raise ValueError("O and dO need q's strides, v needs k's")
    _check_out(L, "L", q.device, torch.float32, (B, H, ql))
    _check_out(sinks, "sinks", q.device, torch.float32, (H,))
    if not _non_overlapping(q.shape, q.stride()):
        q, O, dO = q.contiguous(), O.contiguous(), dO.contiguous()
    if not _non_overlapping(k.shape, k.stride()):
        k, v = k.contiguous(), v.contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dQ = torch.empty_strided(q.shape, q.stride(), dtype=torch.bfloat16, device=q.device)
    dK = torch.empty_strided(k.shape, k.stride(), dtype=torch.bfloat16, device=q.device)
    dV = torch.empty_strided(k.shape, k.stride(), dtype=torch.bfloat16, device=q.device)
    dsinks = torch.empty(H, dtype=torch.float32, device=q.device)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    mptr, mdt, mst = _mask_view(mask, q, k)
    with torch.cuda.device(q.device):
        status = fa_train_bwd_sinks(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), O.data_ptr(), L.data_ptr(), dO.data_ptr(),
            q.stride()[:3], k.stride()[:3], mptr, mdt, mst, B, H, Hkv, ql, kl, D, scale, causal,
            -1 if window is None else window, sinks.data_ptr(), dQ.data_ptr(), dK.data_ptr(),
            dV.data_ptr(), dsinks.data_ptr(), s.cuda_stream)
    if status != 0:
        raise FAError(status, status_string(status))
    return dQ, dK, dV, dsinks


def _fwd_outputs(q, k, v, scale, out, lse, stream):
    """Checks q, k, v and the outputs; returns (O, L, sizes, scale, stream)."""
    import torch

    if not isinstance(q, torch.Tensor):
        raise TypeError("q must be a bfloat16 tensor")
    _check_inputs((("q", q), ("k", k), ("v", v)), q.device)
    B, H, ql, D = q.shape
    Bk, Hkv, kl, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError("k and v must be [B, Hkv, kl, D] with q's B and D")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    O = out if out is not None else torch.empty_like(q)
    L = lse if lse is not None else torch.empty((B, H, ql), dtype=torch.float32, device=q.device)
    _check_out(O, "out", q.device, torch.bfloat16, (B, H, ql, D))
    _check_out(L, "lse", q.device, torch.float32, (B, H, ql))
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    return O, L, (B, H, Hkv, ql, kl, D), scale, s


def train_fwd(q, k, v, mask=None, scale=None, causal=False, out=None, lse=None, stream=None):
    """O, L = train_fwd(q, k, v, mask=None, scale=None, causal=False)

    q: bf16 [B, H, ql, D]; k, v: bf16 [B, Hkv, kl, D] (contiguous, same GPU);
    mask: None or f32 [B, H, ql, kl] additive (natural-log units);
    scale: defaults to 1/sqrt(D); causal: bottom-right aligned.
    Returns O (bf16 [B, H, ql, D]) and L (f32 [B, H, ql]). Enqueued on the
    current stream of q's device (or `stream`, a torch.cuda.Stream).
    """
    return _train_fwd(q, k, v, mask, scale, causal, None, out, lse, stream)


def train_fwd_swa(q, k, v, window, mask=None, scale=None, out=None, lse=None, stream=None):
    """O, L = train_fwd_swa(q, k, v, window, mask=None, scale=None)

    Sliding-window causal forward: key j is visible to query row i iff
    q_abs - window <= j <= q_abs, q_abs = max(kl - ql, 0) + i. Arguments and
    results as for train_fwd (the causal rule is implied).
    """
    return _train_fwd(q, k, v, mask, scale, True, int(window), out, lse, stream)


def _train_fwd(q, k, v, mask, scale, causal, window, out, lse, stream, ex=False,
               mask_layout=None):
    import torch

    if not isinstance(q, torch.Tensor):
        raise TypeError("q must be a bfloat16 tensor")
    _check_inputs((("q", q), ("k", k), ("v", v)), q.device)
    B, H, ql, D = q.shape
    Bk, Hkv, kl, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError("k and v must be [B, Hkv, kl, D] with q's B and D")
    if mask is not None and mask_layout is None:
        if mask.dtype != torch.float32 or not mask.is_contiguous() or mask.device != q.device:
            raise ValueError("mask must be a contiguous float32 tensor on q's device")
        if tuple(mask.shape) != (B, H, ql, kl):
            raise ValueError(f"mask must have shape {(B, H, ql, kl)}")
    if mask is not None and (not _on_gpu(mask) or mask.device != q.device):
        raise ValueError("mask must be on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    O = out if out is not None else torch.empty_like(q)
    L = lse if lse is not None else torch.empty((B, H, ql), dtype=torch.float32, device=q.device)
    _check_out(O, "out", q.device, torch.bfloat16, (B, H, ql, D))
    _check_out(L, "lse", q.device, torch.float32, (B, H, ql))
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    mptr = mask.data_ptr() if mask is not None else 0
    with torch.cuda.device(q.device):
        if ex:
            mdt, sb, sh = mask_layout or (FA_MASK_F32, 0, 0)
            status = fa_train_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), mptr, mdt, sb, sh,
                                     B, H, Hkv, ql, kl, D, scale, causal,
                                     -1 if window is None else window, O.data_ptr(),
                                     L.data_ptr(), s.cuda_stream)
        elif window is None:
            status = fa_train_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), mptr, B, H, Hkv, ql,
                                  kl, D, scale, causal, O.data_ptr(), L.data_ptr(), s.cuda_stream)
        else:
            status = fa_train_fwd_swa(q.data_ptr(), k.data_ptr(), v.data_ptr(), mptr, B, H, Hkv,
                                      ql, kl, D, scale, window, O.data_ptr(), L.data_ptr(),
                                      s.cuda_stream)
    if status != 0:
        raise FAError(status, status_string(status))
    return O, L


def fa_train_bwd(q, k, v, mask, O, L, dO, batch, n_heads, n_kv_heads, ql, kl, head_dim, scale,
                 causal, dQ, dK, dV, stream):
    """The C entry point with raw integer pointers (0 for NULL); returns the status."""
    return lib().fa_train_bwd(q or None, k or None, v or None, mask or None, O or None,
                              L or None, dO or None, batch, n_heads, n_kv_heads, ql, kl, head_dim,
                              float(scale), int(bool(causal)), dQ or None, dK or None, dV or None,
                              stream or None)


def fa_train_bwd_swa(q, k, v, mask, O, L, dO, batch, n_heads, n_kv_heads, ql, kl, head_dim,
                     scale, window, dQ, dK, dV, stream):
    """The C entry point with raw integer pointers (0 for NULL); returns the status."""
    return lib().fa_train_bwd_swa(q or None, k or None, v or None, mask or None, O or None,
                                  L or None, dO or None, batch, n_heads, n_kv_heads, ql, kl,
                                  head_dim, float(scale), int(window), dQ or None, dK or None,
                                  dV or None, stream or None)


def train_bwd_swa(q, k, v, O, L, dO, window, mask=None, scale=None, stream=None):
    """dQ, dK, dV = train_bwd_swa(q, k, v, O, L, dO, window, mask=None, scale=None)

    The backward of train_fwd_swa (same window); otherwise as train_bwd.
    """
    return _train_bwd(q, k, v, O, L, dO, mask, scale, True, int(window), stream)


def fa_train_bwd_ex(q, k, v, mask, mask_dtype, mask_stride_b, mask_stride_h, O, L, dO, batch,
                    n_heads, n_kv_heads, ql, kl, head_dim, scale, causal, window, dQ, dK, dV,
                    stream):
    """The C entry point with raw integer pointers (0 for NULL); returns the status."""
    return lib().fa_train_bwd_ex(q or None, k or None, v or None, mask or None, int(mask_dtype),
                                 int(mask_stride_b), int(mask_stride_h), O or None, L or None,
                                 dO or None, batch, n_heads, n_kv_heads, ql, kl, head_dim,
                                 float(scale), int(bool(causal)), int(window), dQ or None,
                                 dK or None, dV or None, stream or None)


def train_bwd_ex(q, k, v, O, L, dO, mask=None, scale=None, causal=False, window=None,
                 stream=None):
    """dQ, dK, dV = train_bwd_ex(q, k, v, O, L, dO, mask=None, scale=None, causal=False,
                                 window=None)

    The backward of train_fwd_ex with the same mask (float32, bfloat16 or bool,
    [B or 1, H or 1, ql, kl]), causal and window arguments.
    """
    layout = None
    if mask is not None:
        layout = _mask_layout(mask, q, k)
    return _train_bwd(q, k, v, O, L, dO, mask, scale, causal, window, stream, ex=True,
                      mask_layout=layout)


def _mask_layout(mask, q, k):
    """(dtype code, batch stride, head stride) of a mask [B or 1, H or 1, ql, kl]."""
    import torch
    if not isinstance(mask, torch.Tensor) or mask.dtype not in (torch.float32, torch.bfloat16,
                                                                 torch.bool):
        raise ValueError("mask must be float32, bfloat16 or bool")
    B, H, ql, _ = q.shape
    kl = k.shape[2]
    if (mask.dim() != 4 or mask.shape[0] not in (1, B) or mask.shape[1] not in (1, H)
            or tuple(mask.shape[2:]) != (ql, kl)):
        raise ValueError(f"mask must have shape [B or 1, H or 1, {ql}, {kl}]")
    if ql * kl > 0 and ((kl > 1 and mask.stride(3) != 1) or (ql > 1 and mask.stride(2) != kl)):
        raise ValueError("mask rows must be contiguous (strides [.., .., kl, 1])")
    if not _on_gpu(mask) or mask.device != q.device:
        raise ValueError("mask must be on q's device")
    sb = mask.stride(0) if mask.shape[0] > 1 else 0
    sh = mask.stride(1) if mask.shape[1] > 1 else 0
    code = {torch.bfloat16: FA_MASK_BF16, torch.bool: FA_MASK_BOOL}.get(mask.dtype, FA_MASK_F32)
    return code, sb, sh


def train_bwd(q, k, v, O, L, dO, mask=None, scale=None, causal=False, stream=None):
    """dQ, dK, dV = train_bwd(q, k, v, O, L, dO, mask=None, scale=None, causal=False)

    The backward of train_fwd: q, k, v, mask, scale, causal as given to it; O
    and L its outputs; dO (bf16, shaped like O) the upstream gradient. Returns
    bf16 dQ (like q), dK and dV (like k), enqueued on the current stream.
    """
    return _train_bwd(q, k, v, O, L, dO, mask, scale, causal, None, stream)


def _train_bwd(q, k, v, O, L, dO, mask, scale, causal, window, stream, ex=False,
               mask_layout=None):
    import torch

    if not isinstance(q, torch.Tensor):
        raise TypeError("q must be a bfloat16 tensor")
    _check_inputs((("q", q), ("k", k), ("v", v), ("O", O), ("dO", dO)), q.device)
    B, H, ql, D = q.shape
    Bk, Hkv, kl, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError("k and v must be [B, Hkv, kl, D] with q's B and D")
    if O.shape != q.shape or dO.shape != q.shape:
        raise ValueError("O and dO must be shaped like q")
    _check_out(L, "L", q.device, torch.float32, (B, H, ql))
    if mask is not None and not ex:
        if mask.dtype != torch.float32 or not mask.is_contiguous() or mask.device != q.device:
            raise ValueError("mask must be a contiguous float32 tensor on q's device")
        if tuple(mask.shape) != (B, H, ql, kl):
            raise ValueError(f"mask must have shape {(B, H, ql, kl)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dQ, dK, dV = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    mptr = mask.data_ptr() if mask is not None else 0
    with torch.cuda.device(q.device):
        if ex:
            mdt, sb, sh = mask_layout or (FA_MASK_F32, 0, 0)
            status = fa_train_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), mptr, mdt, sb, sh,
                                     O.data_ptr(), L.data_ptr(), dO.data_ptr(), B, H, Hkv, ql, kl,
                                     D, scale, causal, -1 if window is None else window,
                                     dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(), s.cuda_stream)
        elif window is None:
            status = fa_train_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), mptr, O.data_ptr(),
                                  L.data_ptr(), dO.data_ptr(), B, H, Hkv, ql, kl, D, scale,
                                  causal, dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(),
                                  s.cuda_stream)
        else:
            status = fa_train_bwd_swa(q.data_ptr(), k.data_ptr(), v.data_ptr(), mptr,
                                      O.data_ptr(), L.data_ptr(), dO.data_ptr(), B, H, Hkv, ql,
                                      kl, D, scale, window, dQ.data_ptr(), dK.data_ptr(),
                                      dV.data_ptr(), s.cuda_stream)
    if status != 0:
        raise FAError(status, status_string(status))
    return dQ, dK, dV
