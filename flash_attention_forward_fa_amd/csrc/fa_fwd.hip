// fa_fwd.hip - host path and C-ABI entry points of the flash-attention training
// forward (O and L) for AMD MI355X (gfx950): argument checks, the layout of
// strides, decode packing, split-KV workspace, the choice of compensated query
// tiles, and the launches of the kernels of fa_fwd_kernel.h for head dims 64,
// 128 and 256 (80, 96 and 192 are built in fa_fwd_d80.hip, fa_fwd_d96.hip and
// fa_fwd_d192.hip).
#include <hip/hip_runtime.h>

#include <float.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "fa.h"
#include "fa_common.h"
#include "fa_fwd_kernel.h"

namespace {

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Query rows per workgroup of a (DK, DV) pair (of its sliding-window kernels
// when window), 0 for a pair without kernels.
int block_m_of(int dk, int dv, bool window = false) {
  if (dk == dv) {
    switch (dk) {
      case 64: return window ? block_m<64, 64, true>() : block_m<64, 64>();
      case 80: return block_m<80, 80>();
      case 96: return block_m<96, 96>();
      case 128: return block_m<128, 128>();
      case 192: return block_m<192, 192>();
      case 256: return block_m<256, 256>();
    }
    return 0;
  }
  if (dk == 96 && dv == 64) return block_m<96, 64>();
  if (dk == 192 && dv == 128) return block_m<192, 128>();
  return 0;
}
// Head dims of the split-KV, paged and backward paths.
bool base_dim(int d) { return d == 64 || d == 128 || d == 256; }

// Shared host path of every forward entry point; window < 0: none (window >= 0
// requires causal). head_dim is the key width DK, head_dim_v the value width DV
// (V, O and the split-KV partials). The mask is mask_dtype (FA_MASK_F32 / FA_MASK_BF16) with
// batch and head strides in elements; its rows are contiguous (row stride kl).
// Split-KV workspace: partial O (f32, n * rows * D) then, 256-byte aligned,
// partial L (f32, n * rows).
int64_t split_o_bytes(int64_t rows, int head_dim, int64_t n) {
  return (n * rows * head_dim * 4 + 255) / 256 * 256;
}
int64_t split_bytes(int64_t rows, int head_dim, int64_t n) {
  return split_o_bytes(rows, head_dim, n) + n * rows * 4;
}
constexpr int kMaxSplit = 65536;

// Whether the plain tiles' pre-scaled Q is accurate enough at c = |scale|
// log2(e) for key head dim head_dim (see kPlainMaxScaleRootD).
bool plain_scale_ok(float c, int head_dim) {
  return c >= kPlainMinC && c * sqrtf((float)head_dim) <= kPlainMaxScaleRootD * kLog2e;
}

// n_split > 0 selects the split-KV path (no mask, no window) with the given
// workspace.
int train_fwd(const void* q, const void* k, const void* v, const void* mask, int mask_dtype,
              int64_t mask_sb, int64_t mask_sh, int batch, int n_heads, int n_kv_heads, int ql,
              int kl, int head_dim, int head_dim_v, float scale, int causal, int window, void* O,
              float* L, void* stream, int n_split = 0, void* workspace = nullptr,
              size_t workspace_bytes = 0, const int64_t* strides = nullptr,
              int64_t mask_sr = -1, const float* sinks = nullptr) {
  if (batch < 0 || ql < 0 || kl < 0 || n_heads < 1 || n_kv_heads < 1) return FA_ERR_BAD_SIZE;
  if (n_heads % n_kv_heads != 0) return FA_ERR_HEAD_GROUPING;
  if (window >= 0 && !causal) return FA_ERR_WINDOW;
  // a window that hides no key (q_abs - window <= 0 for every row) is the
  // causal problem: it runs the causal kernels, and gives their bits
  if (window >= 0 && (int64_t)window >= (int64_t)std::max(kl - ql, 0) + ql - 1) window = -1;
  const int bm = block_m_of(head_dim, head_dim_v, window >= 0);
  if (bm == 0 || (n_split > 0 && (head_dim != head_dim_v || !base_dim(head_dim))))
    return FA_ERR_HEAD_DIM;
  const int dv = head_dim_v;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (mask && ((mask_dtype != FA_MASK_F32 && mask_dtype != FA_MASK_BF16 &&
                mask_dtype != FA_MASK_BOOL) ||
               mask_sb < 0 || mask_sh < 0))
    return FA_ERR_MASK;
  // element strides (batch, head, row) of Q, K, V, O: given, or contiguous
  int64_t st[12] = {(int64_t)n_heads * ql * head_dim,    (int64_t)ql * head_dim, head_dim,
                    (int64_t)n_kv_heads * kl * head_dim, (int64_t)kl * head_dim, head_dim,
                    (int64_t)n_kv_heads * kl * dv,       (int64_t)kl * dv,       dv,
                    (int64_t)n_heads * ql * dv,          (int64_t)ql * dv,       dv};
  if (strides) {
    for (int i = 0; i < 12; ++i) {
      if (strides[i] < 0) return FA_ERR_STRIDE;
      // 16-byte rows for the vector loads and stores
      if (strides[i] % 8 != 0) return FA_ERR_ALIGNMENT;
      st[i] = strides[i];
    }
    // a K/V tile's rows must lie within a 32-bit buffer offset
    if (st[5] > (1 << 24) || st[8] > (1 << 24) || st[2] > 0x7fffffffLL || st[11] > 0x7fffffffLL)
      return FA_ERR_TOO_LARGE;
    // O is written: no two of its elements may share an address
    const int64_t on[3] = {batch, n_heads, ql};
    if (view_overlaps(st + 9, on, dv)) return FA_ERR_STRIDE;
  }
  const int64_t rows = (int64_t)batch * n_heads * ql;
  if (rows == 0) return FA_OK;
  const bool kv_used = kl > 0;
  if (!q || !O || !L || (kv_used && (!k || !v))) return FA_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(O, 16) || !aligned(L, 4) || (sinks && !aligned(sinks, 4)) ||
      (kv_used && (!aligned(k, 16) || !aligned(v, 16))) ||
      (mask && !aligned(mask, mask_dtype == FA_MASK_BF16 ? 2 : mask_dtype == FA_MASK_BOOL ? 1 : 4)))
    return FA_ERR_ALIGNMENT;
  // One query row per head (decoding), no mask, no window: the layout
  // [B, H, 1, D] of Q, O (and [B, H, 1] of L) is [B, Hkv, H/Hkv, D], so a kv
  // group's query heads are the rows of one packed head and each K/V tile is
  // read once per group. Every such row has q_abs = kl - 1 and sees all kl
  // keys under the causal rule: the packed problem is the non-causal one. The
  // arithmetic of each row is unchanged (rows are computed independently).
  // (with strides: the group's query heads are rows h*q_sh of the packed
  // head, whose stride is G*q_sh; O likewise)
  // (the head strides become row strides, which the kernel holds as int: a
  // head stride beyond that range leaves the heads unpacked)
  // (a sink logit then follows its row: query head g * G + row)
  int sink_group = 1;
  if (ql == 1 && n_heads > n_kv_heads && !mask && window < 0 &&
      st[1] <= 0x7fffffffLL && st[10] <= 0x7fffffffLL) {
    const int G = n_heads / n_kv_heads;
    sink_group = G;
    ql = G;
    n_heads = n_kv_heads;
    causal = 0;
    st[2] = st[1];
    st[1] *= G;
    st[11] = st[10];
    st[10] *= G;
  }
  const int64_t n_qtiles = ((int64_t)ql + bm - 1) / bm;
  const int64_t grid = n_qtiles * batch * n_heads;
  if (grid > 0x7fffffffLL || (int64_t)batch * n_heads > 0x7fffffffLL ||
      (int64_t)kl * std::max(head_dim, dv) * 2 > 0x7fffffffLL)  // one head's K or V must fit a
    return FA_ERR_TOO_LARGE;                                     // buffer descriptor

  FwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.mask = mask;
  a.mask_sb = mask_sb;
  a.mask_sh = mask_sh;
  a.mask_sr = mask_sr < 0 ? kl : (int)mask_sr;
  const int mask_kind = !mask                          ? kNoMask
                        : mask_dtype == FA_MASK_BF16 ? kMaskBF16
                        : mask_dtype == FA_MASK_BOOL ? kMaskBool
                                                     : kMaskF32;
  a.o = static_cast<uint16_t*>(O);
  a.l = L;
  a.B = batch;
  a.H = n_heads;
  a.Hkv = n_kv_heads;
  a.ql = ql;
  a.kl = kl;
  a.group = n_heads / n_kv_heads;
  a.n_qtiles = (int)n_qtiles;
  a.causal_off = kl > ql ? kl - ql : 0;
  // a window reaching past the largest q_abs hides nothing more; clamping it
  // there keeps q_abs - window within int range
  const bool windowed = window >= 0;
  a.window = windowed ? (int)std::min<int64_t>(window, (int64_t)a.causal_off + ql) : 0;
  // Masked keys are carried as raw score -inf and scaled inside the kernel, which
  // needs c > 0; a zero scale is run as the smallest normal one (the scores it
  // produces round to 0 in f32, so the weights are the same uniform ones).
  a.c = fmaxf(fabsf(scale) * kLog2e, FLT_MIN);
  a.q_sign = signbit(scale) ? 0x80008000u : 0u;
  a.q_sb = st[0], a.q_sh = st[1], a.q_sr = (int)st[2];
  a.k_sb = st[3], a.k_sh = st[4], a.k_sr = (int)st[5];
  a.v_sb = st[6], a.v_sh = st[7], a.v_sr = (int)st[8];
  a.o_sb = st[9], a.o_sh = st[10], a.o_sr = (int)st[11];
  a.n_split = 0;
  a.kchunk = 0;
  a.split_plain = 0;
  a.sinks = sinks;
  a.sink_group = sink_group;
  a.ws_o = nullptr;
  a.ws_l = nullptr;
  if (n_split > 0 && kl > 0) {
    // chunks of whole 64-key tiles, each holding at least one key
    const int64_t per = ((int64_t)kl + n_split - 1) / n_split;
    const int64_t kchunk = (per + 63) / 64 * 64;
    const int64_t n_eff = ((int64_t)kl + kchunk - 1) / kchunk;
    if (!workspace) return FA_ERR_NULL_POINTER;
    if (!aligned(workspace, 16)) return FA_ERR_ALIGNMENT;
    if ((int64_t)workspace_bytes < split_bytes(rows, dv, n_eff)) return FA_ERR_SPLIT;
    if (grid * n_eff > 0x7fffffffLL || rows > 0x7fffffffLL) return FA_ERR_TOO_LARGE;
    a.n_split = (int)n_eff;
    a.kchunk = (int)kchunk;
    a.ws_o = static_cast<float*>(workspace);
    a.ws_l = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      split_o_bytes(rows, dv, n_eff));
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  // query tiles whose first row may see fewer than kPreciseKeys keys; every
  // tile when the plain tiles' pre-scaled Q is not used (below)
  int64_t n_short = 0;
  const bool plain_ok = kl > kPlainMinKeys && plain_scale_ok(a.c, head_dim);
  // (split-KV chunks decide per chunk and query tile, in the kernel)
  a.split_plain = a.n_split > 0 && plain_ok;
  if (!plain_ok)
    n_short = n_qtiles;
  else if (windowed && (a.window + 1 < kPreciseKeys ||
                        (ql > kl && (int64_t)ql - 1 > (int64_t)kl + a.window - kPreciseKeys)))
    // every row sees at most window + 1 keys; with ql > kl the last rows
    // (q_abs >= kl) see kl + window - q_abs
    n_short = n_qtiles;
  else if ((causal || windowed) && a.causal_off + 1 < kPreciseKeys)
    n_short = std::min<int64_t>(n_qtiles, (kPreciseKeys - 1 - a.causal_off + bm - 1) / bm);
  const bool cz = causal != 0;
  const int ns = (int)n_short;
  hipError_t err;
  switch (head_dim) {
    case 64: err = dispatch_d<64, 64>(a, cz, windowed, mask_kind, ns, s); break;
    case 128: err = dispatch_d<128, 128>(a, cz, windowed, mask_kind, ns, s); break;
    case 256: err = dispatch_d<256, 256>(a, cz, windowed, mask_kind, ns, s); break;
    case 80: err = fa_fwd_detail::dispatch_d80(a, dv, cz, windowed, mask_kind, ns, s); break;
    case 96: err = fa_fwd_detail::dispatch_d96(a, dv, cz, windowed, mask_kind, ns, s); break;
    default: err = fa_fwd_detail::dispatch_d192(a, dv, cz, windowed, mask_kind, ns, s); break;
  }
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" int fa_train_fwd(const void* q, const void* k, const void* v, const float* mask,
                            int batch, int n_heads, int n_kv_heads, int ql, int kl, int head_dim,
                            float scale, int causal, void* O, float* L, void* stream) {
  const int64_t head = (int64_t)ql * kl;
  return train_fwd(q, k, v, mask, FA_MASK_F32, head * n_heads, head, batch, n_heads, n_kv_heads,
                   ql, kl, head_dim, head_dim, scale, causal, -1, O, L, stream);
}

extern "C" int fa_train_fwd_swa(const void* q, const void* k, const void* v, const float* mask,
                                int batch, int n_heads, int n_kv_heads, int ql, int kl,
                                int head_dim, float scale, int window, void* O, float* L,
                                void* stream) {
  if (window < 0) return FA_ERR_WINDOW;
  const int64_t head = (int64_t)ql * kl;
  return train_fwd(q, k, v, mask, FA_MASK_F32, head * n_heads, head, batch, n_heads, n_kv_heads,
                   ql, kl, head_dim, head_dim, scale, 1, window, O, L, stream);
}

extern "C" unsigned long fa_train_fwd_split_workspace(int batch, int n_heads, int ql, int head_dim,
                                               int n_split) {
  if (batch < 0 || n_heads < 1 || ql < 0 || head_dim < 1 || n_split < 1 || n_split > kMaxSplit)
    return 0;
  return (unsigned long)split_bytes((int64_t)batch * n_heads * ql, head_dim, n_split);
}

extern "C" int fa_train_fwd_split(const void* q, const void* k, const void* v, int batch,
                                  int n_heads, int n_kv_heads, int ql, int kl, int head_dim,
                                  float scale, int causal, int n_split, void* workspace,
                                  unsigned long workspace_bytes, void* O, float* L, void* stream) {
  if (n_split < 1 || n_split > kMaxSplit) return FA_ERR_SPLIT;
  return train_fwd(q, k, v, nullptr, FA_MASK_F32, 0, 0, batch, n_heads, n_kv_heads, ql, kl,
                   head_dim, head_dim, scale, causal, -1, O, L, stream, n_split, workspace,
                   workspace_bytes);
}

extern "C" int fa_paged_fwd(const void* q, const void* k_cache, const void* v_cache,
                            const int* block_table, const int* seq_lens, int batch, int n_heads,
                            int n_kv_heads, int ql, int n_blocks, int block_size, int max_blocks,
                            int head_dim, float scale, int causal, const float* sinks,
                            int n_split, void* workspace, unsigned long workspace_bytes, void* O,
                            float* L, void* stream) {
  if (batch < 0 || ql < 0 || n_heads < 1 || n_kv_heads < 1 || max_blocks < 0 || n_blocks < 0)
    return FA_ERR_BAD_SIZE;
  if (n_heads % n_kv_heads != 0) return FA_ERR_HEAD_GROUPING;
  if (!base_dim(head_dim)) return FA_ERR_HEAD_DIM;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (block_size < 16 || block_size % 16 != 0) return FA_ERR_PAGED;
  if (n_split < 0 || n_split > kMaxSplit) return FA_ERR_SPLIT;
  const int64_t rows = (int64_t)batch * n_heads * ql;
  if (rows == 0) return FA_OK;
  const int64_t cap = (int64_t)max_blocks * block_size;  // keys a table can address
  if (cap > 0x7fffffffLL) return FA_ERR_TOO_LARGE;
  if (cap > 0 && n_blocks < 1) return FA_ERR_PAGED;
  if (!q || !O || !L || !seq_lens || (cap > 0 && (!k_cache || !v_cache || !block_table)))
    return FA_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(O, 16) || !aligned(L, 4) || !aligned(seq_lens, 4) ||
      (sinks && !aligned(sinks, 4)) ||
      (cap > 0 && (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_table, 4))))
    return FA_ERR_ALIGNMENT;
  // decoding: a kv group's query heads as the rows of one head (as in train_fwd;
  // row r of packed head g takes query head g * G + r's sink)
  int H = n_heads, qlen = ql, cz = causal, sink_group = 1;
  if (ql == 1 && n_heads > n_kv_heads) {
    qlen = n_heads / n_kv_heads;
    H = n_kv_heads;
    cz = 0;
    sink_group = qlen;
  }
  const int bm = block_m_of(head_dim, head_dim);
  const int64_t n_qtiles = ((int64_t)qlen + bm - 1) / bm;
  const int64_t grid = n_qtiles * batch * H;
  if (grid > 0x7fffffffLL || (int64_t)batch * H > 0x7fffffffLL ||
      (int64_t)batch * max_blocks > 0x7fffffffLL)
    return FA_ERR_TOO_LARGE;

  FwdArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.o = static_cast<uint16_t*>(O);
  a.l = L;
  a.B = batch;
  a.H = H;
  a.Hkv = n_kv_heads;
  a.ql = qlen;
  a.kl = (int)cap;
  a.group = H / n_kv_heads;
  a.n_qtiles = (int)n_qtiles;
  a.c = fmaxf(fabsf(scale) * kLog2e, FLT_MIN);
  a.q_sign = signbit(scale) ? 0x80008000u : 0u;
  a.q_sb = (int64_t)H * qlen * head_dim, a.q_sh = (int64_t)qlen * head_dim, a.q_sr = head_dim;
  a.o_sb = a.q_sb, a.o_sh = a.q_sh, a.o_sr = a.q_sr;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.max_blocks = max_blocks;
  a.block_size = block_size;
  a.n_blocks = n_blocks;
  a.sinks = sinks;
  a.sink_group = sink_group;
  // plain tiles where a sequence's rows see enough keys (decided per sequence,
  // query tile and chunk in the kernel), for scales whose pre-scaled Q stays in
  // bf16's normal range
  a.split_plain = plain_scale_ok(a.c, head_dim);
  if (n_split > 0 && cap > 0) {
    const int64_t per = (cap + n_split - 1) / n_split;
    const int64_t kchunk = (per + 63) / 64 * 64;
    const int64_t n_eff = (cap + kchunk - 1) / kchunk;
    if (!workspace) return FA_ERR_NULL_POINTER;
    if (!aligned(workspace, 16)) return FA_ERR_ALIGNMENT;
    if ((int64_t)workspace_bytes < split_bytes(rows, head_dim, n_eff)) return FA_ERR_SPLIT;
    if (grid * n_eff > 0x7fffffffLL || rows > 0x7fffffffLL) return FA_ERR_TOO_LARGE;
    a.n_split = (int)n_eff;
    a.kchunk = (int)kchunk;
    a.ws_o = static_cast<float*>(workspace);
    a.ws_l = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      split_o_bytes(rows, head_dim, n_eff));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err = head_dim == 64    ? dispatch_paged<64>(a, cz != 0, s)
                         : head_dim == 128 ? dispatch_paged<128>(a, cz != 0, s)
                                           : dispatch_paged<256>(a, cz != 0, s);
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" int fa_train_fwd_ex(const void* q, const void* k, const void* v, const void* mask,
                               int mask_dtype, long long mask_stride_b, long long mask_stride_h,
                               int batch, int n_heads, int n_kv_heads, int ql, int kl,
                               int head_dim, float scale, int causal, int window, void* O,
                               float* L, void* stream) {
  return train_fwd(q, k, v, mask, mask_dtype, mask_stride_b, mask_stride_h, batch, n_heads,
                   n_kv_heads, ql, kl, head_dim, head_dim, scale, causal, window < 0 ? -1 : window,
                   O, L, stream);
}

namespace {

// The strided entry points: given or contiguous strides of Q, K, V, O and the mask.
int train_fwd_views(const void* q, const long long* q_strides, const void* k,
                    const long long* k_strides, const void* v, const long long* v_strides,
                    const void* mask, int mask_dtype, const long long* mask_strides, int batch,
                    int n_heads, int n_kv_heads, int ql, int kl, int head_dim, int head_dim_v,
                    float scale, int causal, int window, int n_split, void* workspace,
                    unsigned long workspace_bytes, void* O, const long long* o_strides, float* L,
                    void* stream, const float* sinks = nullptr) {
  if (n_split < 0 || n_split > kMaxSplit) return FA_ERR_SPLIT;
  if (n_split > 0 && window >= 0) return FA_ERR_WINDOW;
  if (n_split > 0 && mask) return FA_ERR_MASK;  // split-KV takes no mask
  const long long mhead = (long long)ql * kl;
  const long long ms[3] = {mask_strides ? mask_strides[0] : mhead * n_heads,
                           mask_strides ? mask_strides[1] : mhead,
                           mask_strides ? mask_strides[2] : kl};
  if (mask && (ms[2] < 0 || ms[2] > 0x7fffffffLL)) return FA_ERR_MASK;
  const long long* given[4] = {q_strides, k_strides, v_strides, o_strides};
  const int dv = head_dim_v;
  const long long hq = (long long)ql * head_dim, hk = (long long)kl * head_dim;
  const long long hv = (long long)kl * dv, ho = (long long)ql * dv;
  const long long dflt[4][3] = {{hq * n_heads, hq, head_dim},
                                {hk * n_kv_heads, hk, head_dim},
                                {hv * n_kv_heads, hv, dv},
                                {ho * n_heads, ho, dv}};
  int64_t st[12];
  for (int t = 0; t < 4; ++t)
    for (int i = 0; i < 3; ++i) st[3 * t + i] = given[t] ? given[t][i] : dflt[t][i];
  return train_fwd(q, k, v, mask, mask_dtype, ms[0], ms[1], batch, n_heads, n_kv_heads, ql, kl,
                   head_dim, dv, scale, causal, window, O, L, stream, n_split, workspace,
                   workspace_bytes, st, ms[2], sinks);
}

}  // namespace

extern "C" int fa_train_fwd_strided(const void* q, const long long* q_strides, const void* k,
                                    const long long* k_strides, const void* v,
                                    const long long* v_strides, const void* mask, int mask_dtype,
                                    const long long* mask_strides, int batch, int n_heads,
                                    int n_kv_heads, int ql, int kl, int head_dim, float scale,
                                    int causal, int window, int n_split, void* workspace,
                                    unsigned long workspace_bytes, void* O,
                                    const long long* o_strides, float* L, void* stream) {
  return train_fwd_views(q, q_strides, k, k_strides, v, v_strides, mask, mask_dtype,
                         mask_strides, batch, n_heads, n_kv_heads, ql, kl, head_dim, head_dim,
                         scale, causal, window, n_split, workspace, workspace_bytes, O, o_strides,
                         L, stream);
}

extern "C" int fa_train_fwd_dv(const void* q, const long long* q_strides, const void* k,
                               const long long* k_strides, const void* v,
                               const long long* v_strides, const void* mask, int mask_dtype,
                               const long long* mask_strides, int batch, int n_heads,
                               int n_kv_heads, int ql, int kl, int head_dim, int head_dim_v,
                               float scale, int causal, int window, const float* sinks,
                               int n_split, void* workspace, unsigned long workspace_bytes,
                               void* O, const long long* o_strides, float* L, void* stream) {
  return train_fwd_views(q, q_strides, k, k_strides, v, v_strides, mask, mask_dtype,
                         mask_strides, batch, n_heads, n_kv_heads, ql, kl, head_dim, head_dim_v,
                         scale, causal, window, n_split, workspace, workspace_bytes, O, o_strides,
                         L, stream, sinks);
}

// The library-held scratch of fa_train_fwd_split_noalloc (split-KV partials
// for callers that cannot allocate): one copy per GPU, in this code object.
// Host code never passes this name to a kernel or a copy: on the host it is a
// stand-in, and the device address comes from hipGetSymbolAddress, resolved
// once per device with that device current and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, or nullptr (unknown device,
// or the runtime could not locate the symbol).
void* current_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();  // leave no sticky error for the caller's next call
      return nullptr;
    }
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" int fa_train_fwd_split_noalloc(const void* q, const void* k, const void* v, int batch,
                                          int n_heads, int n_kv_heads, int ql, int kl,
                                          int head_dim, float scale, int causal, int n_split,
                                          void* O, float* L, void* stream) {
  if (n_split < 1 || n_split > kMaxSplit) return FA_ERR_SPLIT;
  if (batch < 0 || ql < 0 || kl < 0 || n_heads < 1 || n_kv_heads < 1) return FA_ERR_BAD_SIZE;
  if (!base_dim(head_dim)) return FA_ERR_HEAD_DIM;
  const int64_t rows = (int64_t)batch * n_heads * ql;
  void* ws = nullptr;
  if (rows > 0 && kl > 0) {
    // the chunks train_fwd will run, and the partials they need
    const int64_t per = ((int64_t)kl + n_split - 1) / n_split;
    const int64_t kchunk = (per + 63) / 64 * 64;
    const int64_t n_eff = ((int64_t)kl + kchunk - 1) / kchunk;
    if (split_bytes(rows, head_dim, n_eff) > (int64_t)FA_NOALLOC_SCRATCH_BYTES)
      return FA_ERR_SCRATCH;
    ws = current_scratch();
    if (!ws) return FA_ERR_SCRATCH;
  }
  return train_fwd(q, k, v, nullptr, FA_MASK_F32, 0, 0, batch, n_heads, n_kv_heads, ql, kl,
                   head_dim, head_dim, scale, causal, -1, O, L, stream, n_split, ws,
                   (size_t)FA_NOALLOC_SCRATCH_BYTES);
}

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case FA_ERR_BAD_SIZE: return "invalid size (batch, ql, kl < 0 or head counts < 1)";
    case FA_ERR_HEAD_GROUPING: return "n_heads is not a multiple of n_kv_heads";
    case FA_ERR_HEAD_DIM:
      return "unsupported head dims: 64, 128 or 256 everywhere; the forward also takes 80, 96, "
             "192 and (key, value) pairs (96, 64) and (192, 128), without split-KV";
    case FA_ERR_SCALE: return "scale must be finite";
    case FA_ERR_ALIGNMENT:
      return "misaligned tensor (q, k, v, O and a workspace need 16 bytes; L, sinks, tables "
             "and an f32 mask 4, a bf16 mask 2)";
    case FA_ERR_TOO_LARGE: return "problem too large for the kernel's grid or index range";
    case FA_ERR_LAUNCH: return "HIP kernel launch failed";
    case FA_ERR_WINDOW:
      return "sliding window must be >= 0 and comes with causal masking, without split-KV";
    case FA_ERR_MASK:
      return "mask dtype must be FA_MASK_F32, FA_MASK_BF16 or FA_MASK_BOOL, strides >= 0, and "
             "no mask with split-KV";
    case FA_ERR_SPLIT: return "n_split must be in 1..65536 and the workspace large enough";
    case FA_ERR_PAGED: return "block_size must be a positive multiple of 16 and the cache non-empty";
    case FA_ERR_SCRATCH:
      return "the split-KV partials exceed the library's 16 MiB scratch, or the scratch could "
             "not be located on the current device";
    case FA_ERR_STRIDE:
      return "strides must be >= 0, and those of a written tensor must not alias its elements";
    default: return "unknown status";
  }
}
