/*
 * fa.h - C ABI of the flash-attention training forward (and its backward) for
 * AMD MI355X (gfx950).
 *
 * The operation is the forward pass of softmax attention as used in training:
 * it returns the attention output O and, for the backward pass, the per-row
 * natural-log logsumexp L. Its definition is the CPU oracle of the method's
 * page ("mlx-native 0.9.0", tests/test_flash_attn_train.rs, doc comment and
 * section "CPU oracle - forward O + logsumexp L"), the launch parameters are
 * those of that page's FlashAttnTrainParams (section "Test helpers",
 * run_train_fwd), and the causal alignment is the one that oracle uses:
 *
 *   per batch b, query head h, query row i, with kv head g = h / (H / Hkv):
 *     s_j = scale * <q[b,h,i,:], k[b,g,j,:]> + mask[b,h,i,j]    (natural log)
 *     key j is hidden when causal and j > max(kl - ql, 0) + i
 *     L[b,h,i]   = log(sum_j exp(s_j))        over visible keys (-inf if none)
 *     O[b,h,i,:] = sum_j exp(s_j - L[b,h,i]) * v[b,g,j,:]        (0 if none)
 *
 * Tensors are contiguous row-major unless an entry point takes strides
 * (fa_train_fwd_ex and fa_train_bwd_ex for the mask; fa_train_fwd_strided and
 * fa_train_bwd_strided for Q, K, V, O and the gradients), in device memory
 * owned by the caller (the split-KV workspace included).
 * The library allocates nothing, keeps no global mutable state and never
 * synchronises: work is enqueued on `stream` and the call returns.
 */
#ifndef FA_MI355X_FA_H
#define FA_MI355X_FA_H

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL_POINTER = 1,   /* q, k, v, O or L is NULL while its tensor is non-empty
                                  (or a required table, length array or workspace, or
                                  fa_train_bwd_sinks' dsinks with sinks set)          */
    FA_ERR_BAD_SIZE = 2,       /* batch, ql or kl < 0; n_heads or n_kv_heads < 1      */
    FA_ERR_HEAD_GROUPING = 3,  /* n_heads is not a multiple of n_kv_heads              */
    FA_ERR_HEAD_DIM = 4,       /* head dims not supported by the entry point: 64, 128
                                  and 256 everywhere; the unsplit forward entry points
                                  also take 80, 96 and 192, and fa_train_fwd_dv the
                                  (key, value) pairs (96, 64) and (192, 128)          */
    FA_ERR_SCALE = 5,          /* scale is NaN or infinite                              */
    FA_ERR_ALIGNMENT = 6,      /* q, k, v, O or a workspace not 16-byte aligned; L,
                                  sinks, dsinks, a block table or lengths not 4-byte;
                                  a mask not aligned to its element                    */
    FA_ERR_TOO_LARGE = 7,      /* a grid or index would overflow the kernel's limits    */
    FA_ERR_LAUNCH = 8,         /* the HIP launch failed (hipGetLastError)               */
    FA_ERR_WINDOW = 9,         /* window < 0 (fa_train_fwd_swa); window >= 0 without
                                  causal, or with split-KV                              */
    FA_ERR_MASK = 10,          /* unknown mask dtype, a negative mask stride, or a mask
                                  with split-KV                                         */
    FA_ERR_SPLIT = 11,         /* n_split outside 1..65536 (0 allowed where it means no
                                  split), or the workspace smaller than the split needs */
    FA_ERR_PAGED = 12,         /* fa_paged_fwd: block_size not a positive multiple of
                                  16, or no cache blocks for a non-empty table          */
    FA_ERR_STRIDE = 13,        /* the strided entry points (fa_train_*_strided,
                                  fa_train_fwd_dv, fa_train_bwd_sinks): a negative
                                  stride, or the strides of a written tensor (O; dQ,
                                  dK, dV) map two of its elements to one address        */
    FA_ERR_SCRATCH = 14        /* fa_train_fwd_split_noalloc: the split-KV partials
                                  exceed FA_NOALLOC_SCRATCH_BYTES, or the library's
                                  scratch could not be located on the current device  */
};

/* Size of the library-held scratch of fa_train_fwd_split_noalloc (per GPU). */
#define FA_NOALLOC_SCRATCH_BYTES (16ul << 20)

/* Element types of an additive mask (fa_train_fwd_ex). */
enum fa_mask_dtype {
    FA_MASK_F32 = 0,   /* additive, f32                                  */
    FA_MASK_BF16 = 1,  /* additive, bf16                                 */
    FA_MASK_BOOL = 2   /* one byte per key: nonzero visible, zero hidden */
};

/*
 * fa_train_fwd - enqueue one training forward pass.
 *
 *   q     bf16 bits [batch, n_heads,    ql, head_dim]  (device, read)
 *   k     bf16 bits [batch, n_kv_heads, kl, head_dim]  (device, read)
 *   v     bf16 bits [batch, n_kv_heads, kl, head_dim]  (device, read)
 *   mask  f32 [batch, n_heads, ql, kl] additive mask in natural-log units, or
 *         NULL for none (device, read). Entries may be -inf (hidden key); +inf
 *         and NaN are outside the contract.
 *   batch, n_heads, n_kv_heads, ql, kl, head_dim: sizes; n_heads must be a
 *         multiple of n_kv_heads (query head h reads kv head h / (n_heads /
 *         n_kv_heads)); head_dim is 64, 80, 96, 128, 192 or 256 (the widths
 *         of the adjacent SDPA page, "nuvec-core 0.3.0", tests/fast.rs,
 *         attention_kernels_match_the_fallback, and the method's own 64 and
 *         256; 80 computes its last 16 dims with a 16-deep MFMA step).
 *   scale finite softmax scale (usually 1/sqrt(head_dim)); negative allowed.
 *   causal nonzero: key j hidden from query row i when j > max(kl - ql, 0) + i.
 *   O     bf16 bits [batch, n_heads, ql, head_dim] (device, written; no
 *         pre-zeroing needed). A row with no visible key gets +0.
 *   L     f32 [batch, n_heads, ql] natural-log logsumexp (device, written);
 *         -inf for a row with no visible key.
 *   stream hipStream_t to enqueue on (NULL: the default stream).
 *
 * Arguments are validated on the host before any HIP call; on error nothing is
 * enqueued and a nonzero fa_status is returned. batch*ql == 0 is a successful
 * no-op; kl == 0 gives every row O = 0 and L = -inf. Input and output buffers
 * must not overlap. The call never aborts and never synchronises.
 */
int fa_train_fwd(const void *q, const void *k, const void *v, const float *mask, int batch,
                 int n_heads, int n_kv_heads, int ql, int kl, int head_dim, float scale,
                 int causal, void *O, float *L, void *stream);

/*
 * fa_train_fwd_swa - enqueue one training forward pass with sliding-window
 * causal attention.
 *
 * The method's page tests a sliding window by building it as an additive mask
 * ("mlx-native 0.9.0", tests/test_flash_attn_train.rs, section 7,
 * "SLIDING-WINDOW MASK (SWA) PARITY": key j kept for row i iff j <= i and
 * j + window >= i). This entry point applies that band directly, with the
 * causal rule's bottom-right alignment (the same as the page's when ql = kl):
 *
 *   key j is visible to query row i iff  q_abs - window <= j <= q_abs,
 *   q_abs = max(kl - ql, 0) + i,
 *
 * so a row sees at most window + 1 keys; key tiles below the band are never
 * read. Every other argument, the layouts, ownership and outputs are those of
 * fa_train_fwd with causal = 1 (an additive mask, when given, applies on top
 * of the band). A row with no visible key (possible when ql > kl) gets O = 0
 * and L = -inf.
 *
 *   window  >= 0; a window of at least max(kl - ql, 0) + ql - 1 hides nothing
 *           beyond the causal rule.
 *
 * Returns FA_ERR_WINDOW for window < 0, otherwise the statuses of
 * fa_train_fwd. Never aborts, never synchronises, allocates nothing.
 */
int fa_train_fwd_swa(const void *q, const void *k, const void *v, const float *mask, int batch,
                     int n_heads, int n_kv_heads, int ql, int kl, int head_dim, float scale,
                     int window, void *O, float *L, void *stream);

/*
 * fa_train_fwd_ex - the forward with every option: mask element type, a mask
 * broadcast over batch and/or heads, causal or sliding-window masking.
 *
 * The method's page passes its additive mask as bf16 ("mlx-native 0.9.0",
 * tests/test_flash_attn_train.rs, section "Test helpers", run_train_fwd and
 * FlashAttnTrainParams); an adjacent attention API on the pages ("nuvec-core
 * 0.3.0", tests/fast.rs, attention_kernels_match_the_fallback) takes an
 * additive mask of shape [1, H, ql, kl] that every batch shares. Both are
 * accepted here; the operation is the one of fa_train_fwd with
 *
 *   mask[b,h,i,j] = mask[b * mask_stride_b + h * mask_stride_h + i * kl + j]
 *
 *   mask          NULL, or mask elements of type mask_dtype (device, read);
 *                 each (b, h) slice is ql rows of kl contiguous elements.
 *                 bf16 values are widened exactly to f32; a boolean mask (the
 *                 same API's [ql, kl] boolean mask) acts as the additive mask
 *                 0 where the byte is nonzero and -inf where it is zero.
 *   mask_dtype    FA_MASK_F32, FA_MASK_BF16 or FA_MASK_BOOL (ignored when mask
 *                 is NULL).
 *   mask_stride_b, mask_stride_h
 *                 element strides between batches and between heads, >= 0;
 *                 0 broadcasts (e.g. 0 and ql*kl for a [1, H, ql, kl] mask).
 *   causal        as for fa_train_fwd.
 *   window        < 0: none; >= 0: the sliding window of fa_train_fwd_swa
 *                 (requires causal != 0).
 *   all others    as for fa_train_fwd.
 *
 * Alignment: an f32 mask 4 bytes, a bf16 mask 2 bytes, a boolean mask 1. Returns the statuses
 * of fa_train_fwd, FA_ERR_MASK for an unknown dtype or a negative stride,
 * FA_ERR_WINDOW for a window without causal masking. fa_train_fwd(...) is
 * fa_train_fwd_ex with an f32 mask, strides H*ql*kl and ql*kl, window -1.
 */
int fa_train_fwd_ex(const void *q, const void *k, const void *v, const void *mask,
                    int mask_dtype, long long mask_stride_b, long long mask_stride_h, int batch,
                    int n_heads, int n_kv_heads, int ql, int kl, int head_dim, float scale,
                    int causal, int window, void *O, float *L, void *stream);

/*
 * fa_train_fwd_strided - fa_train_fwd_ex on strided views of Q, K, V, O and
 * the mask, such as the sequence-major layout [batch, len, heads,
 * head_dim] that an adjacent attention API on the pages passes as transposed
 * views ("nuvec-core 0.3.0", tests/fast.rs, attention_kernels_match_the_fallback,
 * K and V given as views of [B, L, H, D]).
 *
 *   q_strides, k_strides, v_strides, o_strides
 *               host arrays of 3 element strides each: batch, head, row. Element
 *               (b, h, i, d) of Q is q[b*q_strides[0] + h*q_strides[1] +
 *               i*q_strides[2] + d]; head_dim is contiguous. Every stride is a
 *               multiple of 8 elements (16-byte rows; FA_ERR_ALIGNMENT
 *               otherwise) and >= 0 (FA_ERR_STRIDE); K and V row strides at most
 *               2^24 elements (FA_ERR_TOO_LARGE). NULL: that tensor contiguous.
 *               O's strides must give every element its own address: over
 *               the dimensions of size > 1 sorted by stride, each stride at
 *               least the span of those below it (FA_ERR_STRIDE otherwise).
 *               O must not overlap the inputs.
 *   mask, mask_dtype
 *               as for fa_train_fwd_ex (NULL: none)
 *   mask_strides host array of 3 element strides of the mask: batch, head (0
 *               broadcasts) and row (its keys are contiguous), each >= 0, the
 *               row stride below 2^31 (FA_ERR_MASK); NULL: [batch, n_heads, ql, kl] contiguous. A
 *               mask sliced from a larger buffer has a row stride above kl.
 *   L           f32 [batch, n_heads, ql], contiguous, as for fa_train_fwd.
 *   window      as for fa_train_fwd_ex (< 0: none; >= 0 needs causal).
 *   n_split     0: one launch; >= 1: split-KV with workspace, as for
 *               fa_train_fwd_split (no mask: FA_ERR_MASK; head_dim 64, 128 or
 *               256: FA_ERR_HEAD_DIM).
 *   others      as for fa_train_fwd.
 *
 * With all strides NULL this is fa_train_fwd_ex (or fa_train_fwd_split with
 * n_split >= 1), bit for bit.
 */
int fa_train_fwd_strided(const void *q, const long long *q_strides, const void *k,
                         const long long *k_strides, const void *v, const long long *v_strides,
                         const void *mask, int mask_dtype, const long long *mask_strides,
                         int batch, int n_heads, int n_kv_heads, int ql, int kl, int head_dim,
                         float scale, int causal, int window, int n_split, void *workspace,
                         unsigned long workspace_bytes, void *O, const long long *o_strides,
                         float *L, void *stream);

/*
 * fa_train_fwd_dv - fa_train_fwd_strided for a value head dim that may differ
 * from the key head dim, and with optional attention sinks, as in the
 * adjacent SDPA page's attention API ("nuvec-core 0.3.0",
 * tests/fast.rs, attention_kernels_match_the_fallback: (D, Dv) pairs (96, 64)
 * and (192, 128), and sinks [Hq]). The scores use the key width, the weighted
 * sum the value width:
 *
 *     s_j = scale * <q[b,h,i,:head_dim], k[b,g,j,:head_dim]> + mask[b,h,i,j]
 *     O[b,h,i,:head_dim_v] = sum_j exp(s_j - L[b,h,i]) * v[b,g,j,:head_dim_v]
 *
 *   q    bf16 bits [batch, n_heads,    ql, head_dim]    (strided as q_strides)
 *   k    bf16 bits [batch, n_kv_heads, kl, head_dim]    (strided as k_strides)
 *   v    bf16 bits [batch, n_kv_heads, kl, head_dim_v]  (strided as v_strides)
 *   O    bf16 bits [batch, n_heads,    ql, head_dim_v]  (strided as o_strides)
 *   (head_dim, head_dim_v)
 *        (64, 64), (80, 80), (96, 96), (96, 64), (128, 128), (192, 192),
 *        (192, 128) or (256, 256); FA_ERR_HEAD_DIM otherwise. NULL strides:
 *        that tensor contiguous in its own head dim.
 *   sinks f32 [n_heads] (device, read; 4-byte aligned) or NULL: one logit per
 *        query head, in natural-log units, that joins every row's softmax as
 *        one more term with a zero value (the SDPA page's `sinks [Hq]`, which
 *        it passes without defining; this is the reading their name and shape
 *        fix): L = log(exp(sink_h) + sum_j exp(s_j)), O = sum_j exp(s_j - L) v_j.
 *        A row with no visible key gets O = +0 and L = sink_h. -inf sinks
 *        change nothing. With split-KV the chunks' merge adds the sink once.
 *   n_split, workspace, workspace_bytes
 *        0: one launch; >= 1: split-KV as for fa_train_fwd_strided (no mask,
 *        no window; head_dim_v == head_dim in {64, 128, 256}, else
 *        FA_ERR_HEAD_DIM).
 *   others as for fa_train_fwd_strided (mask, window, L, stream, errors).
 *
 * With head_dim_v == head_dim and no sinks this is fa_train_fwd_strided with
 * the same n_split, bit for bit. Allocates nothing; never synchronises.
 */
int fa_train_fwd_dv(const void *q, const long long *q_strides, const void *k,
                    const long long *k_strides, const void *v, const long long *v_strides,
                    const void *mask, int mask_dtype, const long long *mask_strides, int batch,
                    int n_heads, int n_kv_heads, int ql, int kl, int head_dim, int head_dim_v,
                    float scale, int causal, int window, const float *sinks, int n_split,
                    void *workspace, unsigned long workspace_bytes, void *O,
                    const long long *o_strides, float *L, void *stream);

/*
 * fa_train_fwd_split - the forward of fa_train_fwd (no mask, causal or not)
 * with the keys split into chunks that separate workgroups compute: for
 * shapes with few query tiles and many keys (prefill against a long KV cache,
 * decoding), whose plain launch has fewer workgroups than the GPU has CUs.
 *
 * Each chunk c of keys yields, per query row, the softmax over that chunk
 * alone: a normalised partial O_c and its logsumexp L_c (both f32, in the
 * workspace); a second kernel merges them, L = log sum_c exp(L_c),
 * O = sum_c exp(L_c - L) O_c, which is the same softmax over all keys (the
 * L the method's page returns is exactly what makes the merge possible). Every
 * chunk runs the compensated P.V product. O and L are as fa_train_fwd's (O
 * rounded once, from f32, at the merge).
 *
 *   n_split    requested chunks, 1..65536; the keys are cut into chunks of
 *              whole 64-key tiles, ceil(kl / n_split) rounded up, so fewer
 *              chunks may run. The split pays while the plain launch has
 *              fewer workgroups than the GPU has CUs: the plain launch has
 *              batch * n_heads * ceil(ql / R) workgroups (R = 256 query rows
 *              for head_dim 64 and 128, 128 for 256), and batch * n_kv_heads
 *              when ql == 1 (below); about two workgroups per CU in total
 *              (n_split ~ 2 * 256 / that count) was near the fastest on
 *              MI355X, and at one or more per CU the plain call is faster.
 *              At most 16 (packed) query rows with head_dim 64 or 128
 *              (decoding) run a kernel that splits each chunk's keys among
 *              its waves; there about one workgroup per CU and at least 8
 *              chunks was near the fastest, at any batch.
 *
 * Decoding (ql == 1, n_heads > n_kv_heads, no mask, no window; this and the
 * other forward entry points): [B, H, 1, D] is [B, Hkv, H/Hkv, D], so a kv
 * group's query heads run as the rows of one head and each K/V tile is read
 * once per group; each row sees all kl keys either way (same bits).
 *   workspace  device memory of workspace_bytes >= fa_train_fwd_split_workspace
 *              (batch, n_heads, ql, head_dim, n_split), 16-byte aligned, owned by
 *              the caller; its contents on entry do not matter and are
 *              overwritten. Calls that share a workspace must not overlap.
 *   others     as for fa_train_fwd.
 *
 * head_dim is 64, 128 or 256 (FA_ERR_HEAD_DIM otherwise). Returns
 * FA_ERR_SPLIT for n_split outside 1..65536 or a workspace too small,
 * otherwise the statuses of fa_train_fwd. kl == 0 needs no workspace.
 * Two kernel launches; allocates nothing; never synchronises.
 */
int fa_train_fwd_split(const void *q, const void *k, const void *v, int batch, int n_heads,
                       int n_kv_heads, int ql, int kl, int head_dim, float scale, int causal,
                       int n_split, void *workspace, unsigned long workspace_bytes, void *O,
                       float *L, void *stream);

/* Workspace bytes fa_train_fwd_split needs for these sizes (0 if invalid). */
unsigned long fa_train_fwd_split_workspace(int batch, int n_heads, int ql, int head_dim,
                                           int n_split);

/*
 * fa_train_fwd_split_noalloc - fa_train_fwd_split for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the split-KV partials go to a scratch
 * array the library holds instead of a caller workspace. Nothing is
 * allocated, freed or synchronised by the call.
 *
 * The scratch is a device array of FA_NOALLOC_SCRATCH_BYTES (16 MiB) in the
 * library's code object: one copy on every GPU the library runs on, held
 * until the process ends, located on the first call on a GPU. Its bytes are
 * fa_train_fwd_split_workspace(batch, n_heads, ql, head_dim, n_split) of the
 * chunks that run; a call that needs more returns FA_ERR_SCRATCH (e.g.
 * head_dim 128 with batch * n_heads * ql * n_split above 32768 rows) and
 * enqueues nothing. Every call on one GPU shares that GPU's scratch and it
 * keeps the last call's contents (every byte a call reads is written by the
 * same call first, so nothing needs clearing): calls whose kernels may
 * overlap on one GPU (different streams, or other host threads) race on it
 * and must be ordered by the caller. The scratch used is the current
 * device's (hipGetDevice), which must be the device of the tensors and of
 * `stream`.
 *
 * Arguments, outputs and the other statuses are those of fa_train_fwd_split
 * without workspace and workspace_bytes; the kernels and the results are the
 * same bit for bit.
 */
int fa_train_fwd_split_noalloc(const void *q, const void *k, const void *v, int batch,
                               int n_heads, int n_kv_heads, int ql, int kl, int head_dim,
                               float scale, int causal, int n_split, void *O, float *L,
                               void *stream);

/*
 * fa_paged_fwd - the forward against a block-paged KV cache, one key count per
 * sequence (prefill against a cache, decoding).
 *
 * The cache layout and its test are those of an adjacent attention API on
 * the pages ("nuvec-core 0.3.0", tests/fast.rs, the paged helper and
 * paged_attention_equals_contiguous_attention): the result equals the
 * attention of each sequence b over its first seq_lens[b] keys, laid out
 * contiguously. With causal, query row i of sequence b sees keys
 * j <= max(seq_lens[b] - ql, 0) + i (fa_train_fwd's rule per sequence).
 *
 *   q           bf16 [batch, n_heads, ql, head_dim] (device, read)
 *   k_cache,
 *   v_cache     bf16 [n_blocks, n_kv_heads, block_size, head_dim] (device, read)
 *   block_table int32 [batch, max_blocks] (device, read): key position p of
 *               sequence b is row p % block_size of cache block
 *               block_table[b][p / block_size]; entries outside
 *               0..n_blocks-1 are clamped into that range (never an access
 *               outside the cache, but the keys read are then wrong)
 *   seq_lens    int32 [batch] (device, read): keys of each sequence, clamped
 *               to 0..max_blocks*block_size
 *   block_size  a positive multiple of 16 (multiples of 64: one block per
 *               64-key tile; shorter blocks: one per copy instruction)
 *   n_split     0: one launch; >= 1: split-KV with workspace (as for
 *               fa_train_fwd_split, chunks of max_blocks*block_size keys;
 *               workspace size from fa_train_fwd_split_workspace)
 *   sinks       f32 [n_heads] sink logits (device, read; 4-byte aligned) or
 *               NULL, as for fa_train_fwd_dv (one more softmax term per query
 *               head with a zero value; with split-KV the merge adds it once)
 *   O, L        as for fa_train_fwd (a sequence with no key: O = 0, and L =
 *               -inf, or the head's sink)
 *   head_dim    64, 128 or 256 (FA_ERR_HEAD_DIM otherwise)
 *   others      as for fa_train_fwd; no mask, no window.
 *
 * Sequences of more than 256 keys run plain tiles where every row of a query
 * tile (chunk) sees none or at least 128 of the keys, as fa_train_fwd does.
 * Returns FA_ERR_PAGED for a bad
 * block_size or an empty cache behind a non-empty table, FA_ERR_SPLIT as for
 * fa_train_fwd_split, otherwise the statuses of fa_train_fwd. Never
 * synchronises, allocates nothing.
 */
int fa_paged_fwd(const void *q, const void *k_cache, const void *v_cache, const int *block_table,
                 const int *seq_lens, int batch, int n_heads, int n_kv_heads, int ql, int n_blocks,
                 int block_size, int max_blocks, int head_dim, float scale, int causal,
                 const float *sinks, int n_split, void *workspace, unsigned long workspace_bytes,
                 void *O, float *L, void *stream);

/*
 * fa_train_bwd - enqueue the training backward pass of the same attention.
 *
 * Computes the gradients of a loss with upstream gradient dO = dLoss/dO, as
 * the FA-2 backward oracle of the method's page does ("mlx-native 0.9.0",
 * tests/test_flash_attn_train.rs, section "Phase 2 - backward kernel
 * helpers", sdpa_backward_reference_f32), with the forward's causal rule:
 *
 *   P_ij  = exp(s_ij - L_i)  (s_ij as in fa_train_fwd; 0 for a hidden key)
 *   D_i   = sum_d O_id dO_id,   dS_ij = P_ij (dO_i . v_j - D_i)
 *   dQ_i  = scale * sum_j dS_ij k_j,   dK_j = scale * sum_i dS_ij q_i,
 *   dV_j  = sum_i P_ij dO_i      (dK, dV summed over every query head of a
 *                                  kv head's group)
 *
 *   q, k, v, mask, batch .. causal: as for fa_train_fwd (same meaning, same
 *         layouts and constraints), with head_dim 64, 128 or 256
 *         (FA_ERR_HEAD_DIM otherwise).
 *   O     bf16 bits [batch, n_heads, ql, head_dim]: the forward's output (read).
 *   L     f32 [batch, n_heads, ql]: the forward's logsumexp (read); -inf rows
 *         (no visible key) give zero gradients.
 *   dO    bf16 bits [batch, n_heads, ql, head_dim] (read).
 *   dQ    bf16 bits [batch, n_heads, ql, head_dim] (written, fully).
 *   dK    bf16 bits [batch, n_kv_heads, kl, head_dim] (written, fully).
 *   dV    bf16 bits [batch, n_kv_heads, kl, head_dim] (written, fully).
 *   stream hipStream_t to enqueue on (NULL: the default stream).
 *
 * Three kernel launches on `stream`: per query row, L log2(e) and -D_i into
 * the first 8 bytes of the row's dQ memory (dQ serves as scratch until the
 * last launch overwrites it), then dK and dV, then dQ; no atomics, so the
 * result is deterministic. Same validation and status codes as fa_train_fwd
 * (all of q, k, v, O, L, dO, dQ, dK, dV are required for non-empty tensors;
 * 16-byte alignment for the bf16 buffers). The library allocates nothing and
 * never synchronises. Buffers must not overlap.
 */
int fa_train_bwd(const void *q, const void *k, const void *v, const float *mask, const void *O,
                 const float *L, const void *dO, int batch, int n_heads, int n_kv_heads, int ql,
                 int kl, int head_dim, float scale, int causal, void *dQ, void *dK, void *dV,
                 void *stream);

/*
 * fa_train_bwd_swa - the backward of fa_train_fwd_swa: the gradients of the
 * sliding-window causal attention (key j visible to query row i iff
 * q_abs - window <= j <= q_abs, q_abs = max(kl - ql, 0) + i). Arguments,
 * layouts, outputs and statuses are those of fa_train_bwd with causal = 1 and
 * `window` in its place (FA_ERR_WINDOW for window < 0); O and L must come from
 * fa_train_fwd_swa with the same window. Only the key/query tiles inside the
 * band are read.
 */
int fa_train_bwd_swa(const void *q, const void *k, const void *v, const float *mask,
                     const void *O, const float *L, const void *dO, int batch, int n_heads,
                     int n_kv_heads, int ql, int kl, int head_dim, float scale, int window,
                     void *dQ, void *dK, void *dV, void *stream);

/*
 * fa_train_bwd_ex - the backward of fa_train_fwd_ex: the same mask options
 * (mask_dtype, batch/head strides, broadcast), causal and window arguments,
 * with the meaning given for fa_train_fwd_ex; O and L must come from
 * fa_train_fwd_ex with the same options. Other arguments, outputs and
 * statuses as for fa_train_bwd, plus FA_ERR_MASK and FA_ERR_WINDOW as for
 * fa_train_fwd_ex. fa_train_bwd(...) is fa_train_bwd_ex with an f32 mask,
 * strides H*ql*kl and ql*kl, window -1.
 */
int fa_train_bwd_ex(const void *q, const void *k, const void *v, const void *mask,
                    int mask_dtype, long long mask_stride_b, long long mask_stride_h,
                    const void *O, const float *L, const void *dO, int batch, int n_heads,
                    int n_kv_heads, int ql, int kl, int head_dim, float scale, int causal,
                    int window, void *dQ, void *dK, void *dV, void *stream);

/*
 * fa_train_bwd_strided - the backward of fa_train_fwd_strided: the tensors
 * may be strided views with head_dim contiguous, in two layouts, and the
 * mask a strided view as for fa_train_fwd_strided.
 *
 *   q_strides   host array of 3 element strides (batch, head, row) shared by
 *               Q, O, dO and dQ (the gradient is written in Q's layout);
 *               NULL: contiguous [batch, n_heads, ql, head_dim]
 *   kv_strides  the same for K, V, dK and dV; NULL: contiguous
 *   mask, mask_dtype, mask_strides
 *               as for fa_train_fwd_strided (NULL mask: none)
 *   L           f32 [batch, n_heads, ql], contiguous
 *   window      as for fa_train_bwd_ex (< 0: none; >= 0 needs causal)
 *   others      as for fa_train_bwd.
 *
 * Strides are multiples of 8 elements (FA_ERR_ALIGNMENT otherwise) and >= 0
 * (FA_ERR_STRIDE); row strides at most 2^24 elements (FA_ERR_TOO_LARGE).
 * Since the gradients are written with these strides, each triple must give
 * every element its own address (over the dimensions of size > 1 sorted by
 * stride, each stride at least the span of those below it), else
 * FA_ERR_STRIDE: inputs expanded over a dimension (stride 0) must be passed
 * as a copy. The gradients must not overlap the inputs. With all strides NULL
 * this is fa_train_bwd_ex, bit for bit.
 */
int fa_train_bwd_strided(const void *q, const void *k, const void *v, const void *O,
                         const float *L, const void *dO, const long long *q_strides,
                         const long long *kv_strides, const void *mask, int mask_dtype,
                         const long long *mask_strides, int batch, int n_heads, int n_kv_heads,
                         int ql, int kl, int head_dim, float scale, int causal, int window,
                         void *dQ, void *dK, void *dV, void *stream);

/*
 * fa_train_bwd_sinks - the backward of fa_train_fwd_dv with attention sinks
 * (head_dim_v == head_dim): dQ, dK and dV as fa_train_bwd_strided, and the
 * gradient of each query head's sink logit.
 *
 * The sink is one more term of every row's softmax with a zero value (the
 * reading fa_train_fwd_dv states for the adjacent SDPA page's `sinks [Hq]`).
 * O_i depends on sink_h only through L_i, whose derivative is the sink's own
 * weight p_i = exp(sink_h - L_i), so dO_i/dsink_h = -p_i O_i and
 *
 *   dsinks[h] = -sum over every batch b and row i of head h of p_i D_i,
 *               D_i = sum_d O_id dO_id.
 *
 * dQ, dK and dV need nothing more than the forward's L (which includes the
 * sinks): the sink has no value, so it adds nothing to dP or D.
 *
 *   sinks   f32 [n_heads] (device, read; 4-byte aligned), the logits the
 *           forward used, or NULL (then this is fa_train_bwd_strided and
 *           dsinks is not touched)
 *   dsinks  f32 [n_heads] (device, written fully, also when batch * ql = 0;
 *           4-byte aligned); required when sinks is set (FA_ERR_NULL_POINTER)
 *   L       the forward's logsumexp with the same sinks
 *   others  as for fa_train_bwd_strided.
 *
 * One more launch than fa_train_bwd_strided: after the rows pass has put each
 * row's term p_i (-D_i) into its dQ memory, one workgroup per head sums them
 * in a fixed order, so dsinks is deterministic too. Allocates nothing; never
 * synchronises.
 */
int fa_train_bwd_sinks(const void *q, const void *k, const void *v, const void *O,
                       const float *L, const void *dO, const long long *q_strides,
                       const long long *kv_strides, const void *mask, int mask_dtype,
                       const long long *mask_strides, int batch, int n_heads, int n_kv_heads,
                       int ql, int kl, int head_dim, float scale, int causal, int window,
                       const float *sinks, void *dQ, void *dK, void *dV, float *dsinks,
                       void *stream);

/* Static, human-readable name of a status code (never NULL). */
const char *fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_FA_H */
