// fa_fwd_kernel.h - the flash-attention training forward kernel (O and L) for
// AMD MI355X (gfx950), templated on the key and value head dims.
//
// What is computed is fixed by the CPU oracle of the method's page
// ("mlx-native 0.9.0", tests/test_flash_attn_train.rs, doc comment and section
// "CPU oracle - forward O + logsumexp L"): per query row, base-2 scores
// s = scale*log2(e)*<q,k> (+ log2(e)*mask), bottom-right causal masking with the
// offset max(kl - ql, 0), p = exp2(s - m), L = m*ln2 + ln(sum p),
// O = sum(p v) / sum p, and O = 0, L = -inf for a row with no visible key. The
// kernel reaches the same values tile by tile with an online (streaming)
// softmax over key tiles.
//
// Head dims: keys and queries DK, values and O DV, (DK, DV) one of (64, 64),
// (80, 80), (96, 96), (96, 64), (128, 128), (192, 192), (192, 128) and
// (256, 256), the shapes of the adjacent SDPA page ("nuvec-core 0.3.0",
// tests/fast.rs, attention_kernels_match_the_fallback) and the method's own
// 64 and 256.
//
// Work decomposition: one workgroup of 8 waves per (batch, head, query tile);
// each wave owns 32 query rows (two blocks of 16; DK up to 128) or 16 rows
// (DK 192 and 256).
// Per key tile, K and V are copied from HBM straight into LDS
// (buffer_load_dwordx4 ... lds, no VGPR staging) into one of two buffers while
// the previous tile is being computed. Every wave then computes, with
// v_mfma_f32_16x16x32_bf16,
//   S^T = K Q^T     (K rows read from LDS with ds_read_b128; a last 16 dims,
//                    DK = 80, with v_mfma_f32_16x16x16_bf16 and ds_read_b64)
//   O^T += V^T P^T  (V^T read from the row-major V tile with ds_read_b64_tr_b16)
// so that in both products a lane holds one query row per 16-row block: row
// max, row sum and rescale are per-lane scalars after a reduction over the
// four 16-lane groups (v_permlane32_swap, v_permlane16_swap).
//
// Sliding window (the same page, section 7, where it is built as an additive
// mask): key j is visible to row i iff q_abs - window <= j <= q_abs, q_abs =
// max(kl - ql, 0) + i. The WINDOW variants skip the key tiles below the band
// and mask only the tiles that cross one of its edges.
//
// Accuracy: P enters the bf16 MFMA rounded to bf16. Where that is not accurate
// enough the product is compensated (a second MFMA with P's bf16 remainder):
// for query tiles whose rows may see fewer than 128 keys, and for rows whose
// plain result has some |O| >= 1, which their workgroup computes again.
#pragma once

#include <hip/hip_runtime.h>

#include <float.h>
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_common.h"

namespace fa_fwd_detail {

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const void* mask;          // f32, bf16 or bool bytes (the kernel's MASK), or null
  int64_t mask_sb, mask_sh;  // mask strides of batch and head, in elements (0: broadcast)
  int mask_sr;               // mask row stride, in elements (kl: rows contiguous)
  uint16_t* o;
  float* l;
  int B, H, Hkv, ql, kl;
  int group;       // H / Hkv
  int n_qtiles;    // ceil(ql / rows per workgroup)
  int qt_base;     // this launch computes query tiles [qt_base, qt_base + qt_count)
  int qt_count;
  int n_precise;   // kMixed: query tiles below this run compensated
  int split_plain; // split-KV and paged: chunks (or, unsplit, the key range of a paged
                   // sequence) may run plain tiles; else every tile compensated
  const float* sinks;  // f32 sink logits (natural log) of the query heads, or null
  int sink_group;      // 1: head h's sink is sinks[h]; G > 1 (query heads packed as the
                       // G rows of kv head h): row r's is sinks[h * G + r]
  int causal_off;  // max(kl - ql, 0)
  int window;      // WINDOW variants: keys below q_abs - window are hidden
  int n_split;     // kSplit: key chunks per query tile (grid factor)
  int kchunk;      // kSplit: keys per chunk (a multiple of the key tile)
  float* ws_o;     // kSplit: partial O, f32 [n_split, B, H, ql, DV]
  float* ws_l;     // kSplit: partial L, f32 [n_split, B, H, ql]
  const int* block_table;  // paged: int32 [B, max_blocks], block of each block_size keys
  const int* seq_lens;     // paged: int32 [B], keys of each sequence
  int max_blocks, block_size, n_blocks;  // paged: table width, keys per block, cache blocks
  float c;         // |scale| * log2(e), at least FLT_MIN
  uint32_t q_sign; // 0x80008000 flips the sign of both bf16 halves (scale < 0)
  // element strides of batch, head and row (head_dim is contiguous) of Q, K,
  // V and O; L is always contiguous [B, H, ql]
  // (row strides are at most 2^24 elements for K and V, 2^31 - 1 for Q and O)
  int64_t q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;
  int q_sr, k_sr, v_sr, o_sr;
};

// The forward launches of the key widths built in translation units of their
// own (80, 96, 192), for value width dv; hipErrorInvalidValue for a pair they
// do not hold. Arguments as dispatch_d below.
hipError_t dispatch_d80(const FwdArgs& a, int dv, bool causal, bool window, int mask, int n_short,
                        hipStream_t stream);
hipError_t dispatch_d96(const FwdArgs& a, int dv, bool causal, bool window, int mask, int n_short,
                        hipStream_t stream);
hipError_t dispatch_d192(const FwdArgs& a, int dv, bool causal, bool window, int mask,
                         int n_short, hipStream_t stream);

}  // namespace fa_fwd_detail

namespace {

using fa_fwd_detail::FwdArgs;

// Per (key head dim DK, value head dim DV): W waves per workgroup, QB 16-row
// query blocks per wave, BN keys per tile and WPE waves per SIMD of the mixed
// kernel. Eight waves (two per SIMD) share each K/V tile copy, which halves
// the copy traffic per flop against four (measured faster for both).
//   64:  2 blocks (32 rows per wave, 256 per workgroup), 64-key tiles.
//   256: 1 block (16 rows per wave, 128 per workgroup), 64-key tiles (two
//        32 KiB stages of K and V: one workgroup per CU); the O accumulator
//        of 16 rows x 256 dims is 64 registers per lane. 64-key tiles halve
//        the barriers per key against 32 (measured 5% faster).
//   128: 2 blocks (32 rows per wave, 256 per workgroup), 64-key tiles; the O
//        accumulator of 32 rows x 128 dims is 64 registers per lane, two waves
//        per SIMD.
// The other widths follow the nearest of these: 80 and 96 (with DV 80, 96 or
// 64) as 128, 192 (with DV 192 or 128) as 256.
template <int DK, int DV> struct Cfg;
template <> struct Cfg<64, 64> { static constexpr int W = 8, QB = 2, BN = 64, WPE = 4; };
template <> struct Cfg<128, 128> { static constexpr int W = 8, QB = 2, BN = 64, WPE = 2; };
template <> struct Cfg<256, 256> { static constexpr int W = 8, QB = 1, BN = 64, WPE = 2; };
template <> struct Cfg<80, 80> { static constexpr int W = 8, QB = 2, BN = 64, WPE = 2; };
template <> struct Cfg<96, 96> { static constexpr int W = 8, QB = 2, BN = 64, WPE = 2; };
template <> struct Cfg<96, 64> { static constexpr int W = 8, QB = 2, BN = 64, WPE = 2; };
template <> struct Cfg<192, 192> { static constexpr int W = 8, QB = 1, BN = 64, WPE = 2; };
template <> struct Cfg<192, 128> { static constexpr int W = 8, QB = 1, BN = 64, WPE = 2; };
// The sliding-window kernels may use their own shape: with head_dim 64, 4-wave
// workgroups of 128 rows, whose union of the rows' key bands is closer to each
// row's own band than for 256 rows (measured 7% faster at a window of 1024).
template <int DK, int DV, bool WINDOW> struct KCfg : Cfg<DK, DV> {};
template <> struct KCfg<64, 64, true> { static constexpr int W = 4, QB = 2, BN = 64, WPE = 4; };
template <int DK, int DV, bool WINDOW = false> constexpr int block_m() {
  return KCfg<DK, DV, WINDOW>::W * 16 * KCfg<DK, DV, WINDOW>::QB;
}

// Query tiles with a row that may see fewer keys than this (a property of
// their position) are computed with the compensated P.V product (P split into
// a bf16 high part and a bf16 remainder) from the start.
constexpr int kPreciseKeys = 128;
// Plain tiles (bf16 P, Q pre-scaled by c = |scale| log2(e) in bf16) run only
// for problems of more than kPlainMinKeys keys, where the tolerance is 1e-2
// (pre-scaling moves L by up to ~2e-3 and O by up to ~2e-3 before its own
// rounding on the training workloads), for c >= kPlainMinC (c * q stays
// normal in bf16) and for |scale| * sqrt(head_dim) <= kPlainMaxScaleRootD:
// the rounding of c * q moves each base-2 score by about 2^-9 c sqrt(D) |q||k|,
// so at three times the usual 1/sqrt(D) a concentrated softmax's O moved by
// 1.5e-2. Everything else runs compensated, with Q exact.
constexpr int kPlainMinKeys = 256;
constexpr float kPlainMinC = 0x1p-64f, kPlainMaxScaleRootD = 1.5f;
// After a plain pass, a row is recomputed compensated when some |O| element
// reaches this: one bf16 rounding step of O is then 2^-7 or more, so the
// error bf16(P) leaves in O before its own rounding (about 2^-10 at most on
// the workloads) can move it by a step larger than 5e-3. Below it a moved
// rounding costs at most 2^-8. (L needs no such check: bf16(P) changes the
// row sum by a relative 2^-9 at most.)
constexpr float kRecheckO = 1.0f;
// Operand groups (4 MFMAs each) whose LDS reads are in flight ahead of the
// MFMAs in the wide (D > 128) products. (Two ran no faster for D=256 and use
// 249 VGPRs; three spill.)
constexpr int kWidePrefetch = 1;
// The max used in exp2 is only raised when a tile's max exceeds it by more
// than this (base-2 units): P <= 2^kLazy and O is rarely rescaled.
constexpr float kLazy = 8.0f;

// Kernel modes. In the mixed kernel (kMixed) the query tiles below
// n_precise (those with a row that may see fewer than kPreciseKeys keys) run
// the compensated P.V product; the others run the bf16-P product, and when
// some of their rows need the compensated product the workgroup runs the tile
// again, compensated, for those rows only. The compensated kernel (kAll)
// computes every row of every tile compensated (the masked forward).
// In the split-KV kernel (kSplit) a workgroup computes one key chunk of its
// query tile, compensated, and writes the chunk's normalised partial O and its
// logsumexp to a workspace; a combine kernel merges the chunks through L.
// The paged kernels (kPaged, kPagedSplit) read K and V from a block-paged
// cache through a block table, with a key count per sequence; they compute
// every tile compensated, the second one as split-KV partials.
// kPagedBlocks and kPagedBlocksSplit are the same for caches whose blocks are
// shorter than a key tile (block_size a multiple of 16, not of 64).
constexpr int kMixed = 0, kAll = 1, kSplit = 2, kPaged = 3, kPagedSplit = 4, kPagedBlocks = 5,
              kPagedBlocksSplit = 6;





// One query tile of one head: rows qtile * block_m .. of head bh. PRECISE
// selects the compensated P.V product. Without it, a row whose result needs
// that product is not written; its lane's redo[qb] is set instead, and the
// return value tells the whole workgroup whether any of its rows needs it
// (wg_flags: one int per wave). With REDO (and PRECISE), only the rows with
// redo set are computed and written (waves without such a row only take part
// in the tile copies).
template <int DK, int DV, bool CAUSAL, bool WINDOW, int MASK, bool PRECISE, bool REDO,
          bool SPLIT = false, bool PAGED = false, bool SMALL_BLOCKS = false, int QBX = 0>
__device__ __forceinline__ bool fwd_tile(const FwdArgs& a, int qtile, int bh, uint16_t* k0s,
                                         uint16_t* v0s, uint16_t* k1s, uint16_t* v1s,
                                         uint16_t* k2s, uint16_t* v2s, uint16_t* k3s,
                                         uint16_t* v3s,
                                         bool (&redo)[KCfg<DK, DV, WINDOW>::QB], int* wg_flags,
                                         int split = 0) {
  constexpr bool HAS_MASK = MASK != kNoMask;
  static_assert(PRECISE || !HAS_MASK, "the masked forward always runs compensated");
  static_assert(PRECISE || !REDO, "a redo runs compensated");
  static_assert(CAUSAL || !WINDOW, "the sliding window includes the causal rule");
  static_assert(!SPLIT || (!WINDOW && MASK == kNoMask), "split-KV partials: unmasked, no window");
  static_assert(!SPLIT || PAGED || QBX == 0 || PRECISE,
                "the decoding split kernels run compensated");
  static_assert(!PAGED || (!WINDOW && MASK == kNoMask), "paged KV: unmasked, no window");
  static_assert((!SPLIT && !PAGED) || (DK == DV && !kPanels<DK>),
                "split-KV and paged: head dims 64, 128 and 256");
  using C = KCfg<DK, DV, WINDOW>;
  constexpr int BN = C::BN;
  // (QBX: query blocks per wave other than the pair's, for the narrow
  // split-KV kernels of at most 16 query rows: one block, half the work of
  // the one wave that has rows)
  constexpr int kQB = QBX ? QBX : C::QB;
  static_assert(kQB <= C::QB, "redo flags for at most the pair's blocks");
  constexpr int kRowsPerWave = 16 * kQB;
  // The narrow split-KV kernels (at most 16 query rows: decoding) split the
  // keys, not the rows, among the waves: every wave holds the same 16 rows,
  // each takes one 16-key block of a tile, and the waves' partial softmax
  // states are merged through LDS at the end.
  constexpr bool DECODE = QBX == 1 && SPLIT;
  static_assert(!DECODE || (DK == DV && DK <= 128 && !kPanels<DK>), "decode: 64 or 128 dims");
  constexpr int kBlockM = DECODE ? 16 : C::W * kRowsPerWave;
  constexpr int NKB = BN / 16;   // 16-key blocks per tile
  constexpr int NKC = BN / 32;   // 32-key chunks per tile (P.V contraction steps)
  constexpr int NDB = DV / 16;   // 16-dim blocks of O
  constexpr int NDS = DK / 32;   // 32-dim steps of Q.K
  // a last 16-dim step of Q.K (DK = 80), with the 16x16x16 MFMA
  constexpr bool KTAIL = DK % 32 == 16;
  constexpr int NT = 64 * C::W;  // threads per workgroup
  // the wide key dims (one query block per wave): grouped operand reads
  constexpr bool WIDE = DK > 128;
  static_assert(DK % 16 == 0 && DV % 16 == 0 && NDS > 0, "head dims: multiples of 16, >= 32");
  // Plain tiles take Q pre-scaled by c = |scale| log2(e) and rounded to bf16,
  // so that the MFMA yields base-2 scores; their accumulators start at -m
  // (the running max), so exp2 reads the MFMA's output directly. The
  // compensated tiles keep Q exact and scale in f32.
  constexpr bool PS = !PRECISE;

  // (the opaque copy keeps the compiler from hoisting the thread-index
  // arithmetic of both tile variants of the mixed kernel above their branch,
  // where it would stay live, and spill, across both)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  // The wave index is made provably wave-uniform so that every condition
  // derived from it (tile skipping, masking, row selection) compiles to a
  // scalar branch: an MFMA left inside an EXEC-masked region still accumulates
  // (with whatever its operand registers hold) when EXEC is zero.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int c16 = lane & 15;  // query column within a 16-row block / A-operand row
  const int grp = lane >> 4;  // 16-lane group

  const int b = bh / a.H, h = bh % a.H;
  const int g = h / a.group;
  // (paged KV: the sequence's own key count, at most its table's capacity, and
  // its own causal offset)
  const int kl = PAGED ? min(max(load_uniform(a.seq_lens, b), 0),
                             a.max_blocks * a.block_size)
                       : a.kl;
  const int ql = a.ql, off = PAGED ? max(kl - ql, 0) : a.causal_off;
  const int q0 = qtile * kBlockM;
  const int qw0 = DECODE ? q0 : q0 + wave * kRowsPerWave;
  const uint16_t* kp = a.k + b * a.k_sb + g * a.k_sh;
  const uint16_t* vp = a.v + b * a.v_sb + g * a.v_sh;
  // row strides of the K and V sources (a paged cache's rows are contiguous)
  const int k_rs = PAGED ? DK : a.k_sr, v_rs = PAGED ? DV : a.v_sr;

  // ---- key range ----
  // (split-KV: only the keys of chunk `split`, [split*kchunk, (split+1)*kchunk))
  const int k_hi = SPLIT ? (split + 1) * a.kchunk : kl;
  const int last_row = min(q0 + kBlockM, ql) - 1;
  const int kend = min(k_hi, CAUSAL ? min(kl, off + last_row + 1) : kl);
  const int n_kt = (kend + BN - 1) / BN;
  // under a sliding window no row of the workgroup (of the wave) sees a key
  // below off + (its first row) - window: those key tiles are skipped
  const int kt_first = SPLIT ? split * a.kchunk / BN : WINDOW ? max(0, off + q0 - a.window) / BN : 0;
  const bool wave_active = qw0 < ql;
  const int wave_last = min(qw0 + kRowsPerWave, ql) - 1;
  const int wave_kend = min(k_hi, CAUSAL ? min(kl, off + wave_last + 1) : kl);
  const int wave_kt_first =
      SPLIT ? kt_first : WINDOW ? max(0, off + qw0 - a.window) / BN : 0;
  float* lrow_base = a.l + (int64_t)bh * ql;

  bool wave_redo = false;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) wave_redo |= redo[qb];
  const bool compute = wave_active && (!REDO || __any(wave_redo));

  int koff[CopyShape<DK, BN, NT>::ROUNDS], voff[CopyShape<DV, BN, NT>::ROUNDS];
  copy_offsets<DK, BN, NT, true>(tid, koff, k_rs);
  copy_offsets<DV, BN, NT, false>(tid, voff, v_rs);
  // paged KV: when block_size is a multiple of BN a tile lies in one block,
  // table[b][kt*BN / block_size], from row (kt*BN) % block_size, and its copy
  // descriptor covers only the tile's valid rows; shorter blocks (multiples
  // of 16) are looked up per wave instruction (issue_tile_blocks). A table
  // entry outside the cache is clamped into it (wrong keys, never an access
  // outside the cache).
  const int* table_row = PAGED ? a.block_table + (int64_t)b * a.max_blocks : nullptr;
  auto paged_src = [&](const uint16_t* cache, int kt) {
    const int pos = kt * BN;
    int blk = load_uniform(a.block_table, (int64_t)b * a.max_blocks + pos / a.block_size);
    blk = min(max(blk, 0), a.n_blocks - 1);
    return cache + (((int64_t)blk * a.Hkv + g) * a.block_size + pos % a.block_size) * DK;
  };
  auto issue_k = [&](int kt, uint16_t* dst) {
    if constexpr (PAGED) {
      if constexpr (!SMALL_BLOCKS)
        issue_tile<DK, BN, NT, true, true>(paged_src(a.k, kt), 0, min(BN, kl - kt * BN), dst, tid,
                                     64 * wave, koff);
      else
        issue_tile_blocks<DK, BN, NT, true>(a.k, table_row, a.n_blocks, a.Hkv, g, a.block_size,
                                            kt * BN, kl, dst, tid, 64 * wave);
    } else
      issue_tile<DK, BN, NT, true, true>(kp, kt * BN, kl, dst, tid, 64 * wave, koff, k_rs);
  };
  auto issue_v = [&](int kt, uint16_t* dst) {
    if constexpr (PAGED) {
      if constexpr (!SMALL_BLOCKS)
        issue_tile<DV, BN, NT, false, true>(paged_src(a.v, kt), 0, min(BN, kl - kt * BN), dst, tid,
                                      64 * wave, voff);
      else
        issue_tile_blocks<DV, BN, NT, false>(a.v, table_row, a.n_blocks, a.Hkv, g, a.block_size,
                                             kt * BN, kl, dst, tid, 64 * wave);
    } else
      issue_tile<DV, BN, NT, false, true>(vp, kt * BN, kl, dst, tid, 64 * wave, voff, v_rs);
  };
  // Split-KV and paged tiles of up to 128 dims run a four-stage copy pipeline
  // (tile kt in buffer kt % 4, three tiles in flight while one is computed):
  // their workgroups are few per CU and short, and with one tile in flight
  // the copies' latency, not HBM, set their pace.
  constexpr int NSTAGE = (SPLIT || PAGED) && DK <= 128 ? 4 : 2;
  uint16_t* const kst[4] = {k0s, k1s, k2s, k3s};
  uint16_t* const vst[4] = {v0s, v1s, v2s, v3s};
  if constexpr (DECODE) {
    // (the first three tiles, in stages 0 to 2)
    for (int i = 0; i < 3; ++i)
      if (kt_first + i < n_kt) issue_k(kt_first + i, kst[i]);
  } else if constexpr (NSTAGE == 4) {
    for (int i = 0; i < 3; ++i)
      if (kt_first + i < n_kt) issue_k(kt_first + i, kst[(kt_first + i) & 3]);
  } else {
    if (n_kt > kt_first) issue_k(kt_first, (kt_first & 1) ? k1s : k0s);
  }

  // ---- Q^T as the B operand: block qb, step s: row qw0+16qb+c16, dims 32s+8grp.. ----
  // (and in a 16-dim tail step: dims 32 NDS + 4grp ..)
  bf16x8 qop[kQB][NDS];
  bf16x4 qtail[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int qrow = min(qw0 + 16 * qb + c16, ql - 1);
    const uint16_t* qrp = a.q + b * a.q_sb + h * a.q_sh + (int64_t)qrow * a.q_sr;
    const uint16_t* qp = qrp + 8 * grp;
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
      u32x4 raw = *reinterpret_cast<const u32x4*>(qp + 32 * s);
      raw ^= a.q_sign;
      qop[qb][s] = __builtin_bit_cast(bf16x8, raw);
      if constexpr (PS) {
        bf16x8 sc;
#pragma unroll
        for (int e = 0; e < 8; ++e) sc[e] = (__bf16)((float)qop[qb][s][e] * a.c);
        qop[qb][s] = sc;
      }
    }
    if constexpr (KTAIL) {
      typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
      u32x2 raw = *reinterpret_cast<const u32x2*>(qrp + 32 * NDS + 4 * grp);
      raw ^= a.q_sign;
      qtail[qb] = __builtin_bit_cast(bf16x4, raw);
      if constexpr (PS) {
#pragma unroll
        for (int e = 0; e < 4; ++e) qtail[qb][e] = (__bf16)((float)qtail[qb][e] * a.c);
      }
    }
  }

  // m_use: the max used in exp2 (base 2); thr: the tile max above which a
  // tile raises it (m_use + kLazy in raw units; in the plain tiles, whose
  // scores come relative to m_use, kLazy); l_run: this lane's partial row
  // sum. The plain tiles start m_use at 0 (their scores are then the raw
  // ones) and take the first visible key's tile max as it; the compensated
  // ones start at the finite sentinel -FLT_MAX/2.
  float m_use[kQB], thr[kQB], l_run[kQB];
  f32x4 oacc[NDB][kQB];
  const float inv_c = HAS_MASK ? 1.0f : 1.0f / a.c;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    m_use[qb] = PS ? 0.0f : -FLT_MAX / 2.0f;
    thr[qb] = -INFINITY;
    l_run[qb] = 0.0f;
#pragma unroll
    for (int d = 0; d < NDB; ++d) oacc[d][qb] = f32x4{};
  }

  // The wave's own key tiles, and the first of them that needs a mask (the
  // partial last tile, or the causal diagonal of the wave's first row).
  const int n_kw = (compute && wave_kend > 0) ? (wave_kend + BN - 1) / BN : 0;
  int mask_from = HAS_MASK ? 0 : n_kw;
  if (!HAS_MASK) {
    if (kl % BN != 0) mask_from = min(mask_from, kl / BN);
    if (CAUSAL) mask_from = min(mask_from, (off + qw0 + 1) / BN);
  }
  // and the tiles below lo_end, which hold keys that the wave's last row no
  // longer sees (the window's lower edge)
  const int lo_gap = WINDOW ? off + wave_last - a.window : 0;
  const int lo_end = lo_gap > 0 ? (lo_gap + BN - 1) / BN : 0;

  const int lane_c16 = c16, lane_grp = grp;

  // ---- S^T = K Q^T (raw scores, f32) for the tile in ks ----
  auto kread = [&](const uint16_t* ks, int s, int kb) {
    const int r = key_of(kb, lane_c16);
    // (one index off the tile: every LDS address a short GEP chain from its
    // buffer, so that the compiler keeps the buffer's alias scope on the read)
    return *reinterpret_cast<const bf16x8*>(ks + k_step_piece<DK>(r, s, lane_grp));
  };
  // the 16-dim tail step's K operand of key block kb (A of 16x16x16: row c16,
  // dims 4grp .. of the tail)
  auto kread_tail = [&](const uint16_t* ks, int kb) {
    const int r = key_of(kb, lane_c16);
    if constexpr (KTAIL)
      return *reinterpret_cast<const bf16x4*>(ks + k_tail16_piece<DK>(r, lane_grp));
    else
      return bf16x4{};
  };
  auto scores = [&](const uint16_t* ks, f32x4 (&sacc)[NKB][kQB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        if constexpr (PS)
          sacc[kb][qb] = f32x4{-m_use[qb], -m_use[qb], -m_use[qb], -m_use[qb]};
        else
          sacc[kb][qb] = f32x4{};
      }
    if constexpr (!WIDE) {
#pragma unroll
      for (int s = 0; s < NDS; ++s)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const bf16x8 kop = kread(ks, s, kb);
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb)
            sacc[kb][qb] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[qb][s], sacc[kb][qb], 0, 0, 0);
        }
      if constexpr (KTAIL) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const s16x4 kop = __builtin_bit_cast(s16x4, kread_tail(ks, kb));
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb)
            sacc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                kop, __builtin_bit_cast(s16x4, qtail[qb]), sacc[kb][qb], 0, 0, 0);
        }
      }
    } else {
      // DK > 128: K operands in groups of SG dim steps, the reads of group
      // g + kWidePrefetch issued before the MFMAs of group g; sched_barrier
      // keeps that order (and the register use) instead of hoisting every read.
      constexpr int SG = NKB == 2 ? 2 : 1;
      constexpr int NG = NDS / SG;
      constexpr int PD = kWidePrefetch, NR = PD + 1;
      bf16x8 kop[NR][SG][NKB];
#pragma unroll
      for (int p = 0; p < PD && p < NG; ++p)
#pragma unroll
        for (int ss = 0; ss < SG; ++ss)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) kop[p][ss][kb] = kread(ks, p * SG + ss, kb);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g + PD < NG) {
#pragma unroll
          for (int ss = 0; ss < SG; ++ss)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
              kop[(g + PD) % NR][ss][kb] = kread(ks, (g + PD) * SG + ss, kb);
        }
#pragma unroll
        for (int ss = 0; ss < SG; ++ss)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb)
              sacc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  kop[g % NR][ss][kb], qop[qb][g * SG + ss], sacc[kb][qb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- masks of tile kt: tail keys, causal, additive ----
  auto apply_mask = [&](int kt, f32x4 (&sacc)[NKB][kQB]) {
    const int kbase = kt * BN;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const int qrow = qw0 + 16 * qb + c16;
      if constexpr (HAS_MASK) {
        const int64_t mrow =
            b * a.mask_sb + h * a.mask_sh + (int64_t)min(qrow, ql - 1) * a.mask_sr;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kbase + 32 * (kb >> 1) + 8 * grp + 4 * (kb & 1) + i;
            const bool vis = key < kl && (!CAUSAL || key <= off + qrow) &&
                             (!WINDOW || key >= off + qrow - a.window);
            // (the index is clamped so that keys past the end read inside the row)
            const float mv = mask_at<MASK>(a.mask, mrow + min(key, kl - 1));
            sacc[kb][qb][i] = vis ? __builtin_fmaf(sacc[kb][qb][i], a.c, kLog2e * mv) : -INFINITY;
          }
      } else {
        // the last (and, under a window, the first) visible key of the row,
        // relative to this lane's first key of the tile; each score then needs
        // one compare with a constant per edge
        const int last = (CAUSAL ? min(kl - 1, off + qrow) : kl - 1) - kbase - 8 * grp;
        const int first = WINDOW ? off + qrow - a.window - kbase - 8 * grp : 0;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int idx = 32 * (kb >> 1) + 4 * (kb & 1) + i;
            if (idx > last || (WINDOW && idx < first)) sacc[kb][qb][i] = -INFINITY;
          }
      }
    }
  };

  // ---- online softmax (base 2): row max of a tile, lazy raise ----
  // (the decision to raise is taken per row, so a row's result never depends
  // on its neighbours' scores)
  // (the max is compared with thr in raw-score units; c > 0, so
  // max(c*r) == c*max(r))
  // The lane's own part of the row max (16 of the tile's keys for each of its
  // rows) already tells whether the row max exceeds thr; only when some lane
  // of the wave finds that is the max completed over the four 16-lane groups.
  auto part_max = [&](const f32x4 (&sacc)[NKB][kQB], float (&mx)[kQB]) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      mx[qb] = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx[qb] = __builtin_fmaxf(mx[qb], sacc[kb][qb][i]);
    }
    bool raise = false;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) raise |= mx[qb] > thr[qb];
    return raise;
  };
  auto complete_max = [&](float (&mx)[kQB]) {
    if constexpr (kQB == 2) {
      group_max2(mx[0], mx[1]);
    } else {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) mx[qb] = group_max(mx[qb]);
    }
  };
  auto rescale = [&](const float (&mx)[kQB], f32x4 (&sacc)[NKB][kQB]) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const bool r = mx[qb] > thr[qb];
      float m_new, alpha;
      if constexpr (PS) {
        // scores relative to m_use: the new max is m_use + mx, and this
        // tile's scores move down by mx (later tiles start at the new -m_use).
        // A row's first raise may lower m_use (from 0); its sum and O are
        // still 0 then, and alpha is kept at most 1.
        const float shift = r ? mx[qb] : 0.0f;
        m_new = m_use[qb] + shift;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) sacc[kb][qb] -= shift;
        thr[qb] = r ? kLazy : thr[qb];
        alpha = __builtin_amdgcn_exp2f(fminf(-shift, 0.0f));
      } else {
        m_new = r ? (HAS_MASK ? mx[qb] : mx[qb] * a.c) : m_use[qb];
        thr[qb] = r ? (m_new + kLazy) * inv_c : thr[qb];
        alpha = __builtin_amdgcn_exp2f(m_use[qb] - m_new);
      }
      m_use[qb] = m_new;
      l_run[qb] *= alpha;
#pragma unroll
      for (int d = 0; d < NDB; ++d) oacc[d][qb] *= alpha;
    }
  };

  // ---- P = exp2(s - m) in bf16 (+ remainder when compensated), row sums ----
  auto probs = [&](const f32x4 (&sacc)[NKB][kQB], bf16x8 (&phi)[NKC][kQB],
                   bf16x8 (&plo)[NKC][kQB]) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float mneg = -m_use[qb];
      float ls = l_run[qb];
#pragma unroll
      for (int j = 0; j < NKC; ++j) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sv = sacc[2 * j + (e >> 2)][qb][e & 3];
          p[e] = __builtin_amdgcn_exp2f(HAS_MASK ? sv + mneg
                                        : PS     ? sv
                                                 : __builtin_fmaf(sv, a.c, mneg));
          phi[j][qb][e] = (__bf16)p[e];
        }
#pragma unroll
        for (int e = 0; e < 8; e += 2)
          ls = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{phi[j][qb][e], phi[j][qb][e + 1]}, ones, ls,
                                               false);
        if (PRECISE) {
#pragma unroll
          for (int e = 0; e < 8; ++e) plo[j][qb][e] = (__bf16)(p[e] - (float)phi[j][qb][e]);
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            ls = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{plo[j][qb][e], plo[j][qb][e + 1]}, ones,
                                                 ls, false);
        }
      }
      l_run[qb] = ls;
    }
  };

  // ---- O^T += V^T P^T for the tile in vs ----
  // V^T operand of dim block d, key chunk j: dims 16d + c16, keys
  // 32j + 8grp + (0..7), from two transposing reads of four keys each
  auto vread = [&](const uint16_t* vs, int d, int j) {
    s16x4 half[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r = 32 * j + 8 * lane_grp + 4 * t + (lane_c16 >> 2);
      const uint16_t* addr = vs + v_piece<DV>(r, d, lane_c16 & 3);
      half[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)addr);
    }
    return __builtin_bit_cast(bf16x8,
                              __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto pv_mfma = [&](const bf16x8& vop, int d, int j, const bf16x8 (&phi)[NKC][kQB],
                     const bf16x8 (&plo)[NKC][kQB]) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      oacc[d][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, phi[j][qb], oacc[d][qb], 0, 0, 0);
      if (PRECISE)
        oacc[d][qb] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, plo[j][qb], oacc[d][qb], 0, 0, 0);
    }
  };
  auto pv = [&](const uint16_t* vs, const bf16x8 (&phi)[NKC][kQB], const bf16x8 (&plo)[NKC][kQB]) {
    if constexpr (DV <= 128) {
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int j = 0; j < NKC; ++j) pv_mfma(vread(vs, d, j), d, j, phi, plo);
    } else {
      // DV > 128: V operands in groups of DG dim blocks, prefetched
      // kWidePrefetch groups ahead as for K
      constexpr int DG = NKC == 1 ? 4 : 2;
      constexpr int NG = NDB / DG;
      constexpr int PD = kWidePrefetch, NR = PD + 1;
      bf16x8 vop[NR][DG][NKC];
#pragma unroll
      for (int p = 0; p < PD && p < NG; ++p)
#pragma unroll
        for (int dd = 0; dd < DG; ++dd)
#pragma unroll
          for (int j = 0; j < NKC; ++j) vop[p][dd][j] = vread(vs, p * DG + dd, j);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g + PD < NG) {
#pragma unroll
          for (int dd = 0; dd < DG; ++dd)
#pragma unroll
            for (int j = 0; j < NKC; ++j)
              vop[(g + PD) % NR][dd][j] = vread(vs, (g + PD) * DG + dd, j);
        }
#pragma unroll
        for (int dd = 0; dd < DG; ++dd)
#pragma unroll
          for (int j = 0; j < NKC; ++j) pv_mfma(vop[g % NR][dd][j], g * DG + dd, j, phi, plo);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- the key loop ----
  // One tile per step: wait for its copy, start the next one, compute it.
  // Where registers allow (PAIRED), the steps come in pairs with fixed buffer
  // roles (even tiles in buffer 0, odd tiles in buffer 1), so that the
  // compiler can tell the LDS reads of a tile from the copy of the next one in
  // flight into the other buffer: with the buffer chosen at run time it makes
  // every wave wait for that copy before its V^T reads (measured: D=64 4k
  // causal 326 -> 316 us, D=256 8k 1106 -> 1065 us). With fixed buffers the
  // compiler keeps the addresses of both buffers in registers, which spills
  // in the sliding-window, split-KV and paged kernels and in the compensated
  // tiles of the mixed kernel (the short first tiles and the rare redo):
  // those keep one step per iteration.
  constexpr bool PAIRED = !WINDOW && !SPLIT && !PAGED && (!PRECISE || HAS_MASK);
  auto step = [&](int kt, const uint16_t* kc, const uint16_t* vc, uint16_t* kn, uint16_t* vn) {
    wait_vmem();
    __syncthreads();
    if (kt + 1 < n_kt) {
      issue_k(kt + 1, kn);
      issue_v(kt + 1, vn);
    }
    if (kt >= wave_kt_first && kt < n_kw) {
      // A wave issuing its MFMA blocks gets a raised priority (s_setprio), so
      // it is not held back behind the other waves' VALU work; measured best
      // around the P.V block for D=64 and around both blocks for D=256.
      f32x4 s[NKB][kQB];
      if (WIDE) set_prio<2>();
      scores(kc, s);
      if (WIDE) set_prio<0>();
      if (kt >= mask_from || (WINDOW && kt < lo_end)) apply_mask(kt, s);
      float mx[kQB];
      if (__any(part_max(s, mx))) {
        complete_max(mx);
        rescale(mx, s);
      }
      bf16x8 phi[NKC][kQB], plo[NKC][kQB];
      probs(s, phi, plo);
      set_prio<2>();
      pv(vc, phi, plo);
      set_prio<0>();
    }
  };
  if constexpr (DECODE) {
    for (int i = 0; i < 3; ++i)
      if (kt_first + i < n_kt) issue_v(kt_first + i, vst[i]);
  } else if constexpr (NSTAGE == 4) {
    for (int i = 0; i < 3; ++i)
      if (kt_first + i < n_kt) issue_v(kt_first + i, vst[(kt_first + i) & 3]);
  } else {
    if (n_kt > kt_first) issue_v(kt_first, (kt_first & 1) ? v1s : v0s);
  }
  if constexpr (DECODE) {
    // One tile per step, wave w < 4 taking its keys 16 w .. (the copies, not
    // the arithmetic, set the pace here: the four other waves only copy).
    // Tile kt_first + i sits in stage i & 3; three tiles are in flight while
    // one is computed, and a step's copy goes to the stage the previous step
    // read.
    constexpr int R = CopyShape<DK, BN, NT>::ROUNDS + CopyShape<DV, BN, NT>::ROUNDS;
    const int kb_w = wave & 3;
    const int row = qw0 + c16;
    float& mu = m_use[0];
    float& th = thr[0];
    float& lr = l_run[0];
    auto tile_work = [&](int kt, const uint16_t* ks, const uint16_t* vs) {
      // S^T of the block's 16 keys: lane (c16, grp) holds keys 4 grp + e of row c16
      f32x4 sacc = {};
#pragma unroll
      for (int st = 0; st < NDS; ++st) {
        const bf16x8 kop =
            *reinterpret_cast<const bf16x8*>(ks + k_step_piece<DK>(16 * kb_w + c16, st, grp));
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[0][st], sacc, 0, 0, 0);
      }
      const int key0 = kt * BN + 16 * kb_w + 4 * grp;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = key0 + e;
        if (!(key < kl && (!CAUSAL || key <= off + row))) sacc[e] = -INFINITY;
      }
      float mx = __builtin_fmaxf(__builtin_fmaxf(sacc[0], sacc[1]), __builtin_fmaxf(sacc[2], sacc[3]));
      if (__any(mx > th)) {
        mx = group_max(mx);
        const bool r = mx > th;
        const float m_new = r ? mx * a.c : mu;
        th = r ? (m_new + kLazy) * inv_c : th;
        const float alpha = __builtin_amdgcn_exp2f(mu - m_new);
        mu = m_new;
        lr *= alpha;
#pragma unroll
        for (int d = 0; d < NDB; ++d) oacc[d][0] *= alpha;
      }
      // P = exp2(s - m) as bf16 and its bf16 remainder, and the row sum
      bf16x4 ph, pl;
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e], a.c, -mu));
        ph[e] = (__bf16)p;
        pl[e] = (__bf16)(p - (float)ph[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        lr = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{ph[e], ph[e + 1]}, ones, lr, false);
        lr = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pl[e], pl[e + 1]}, ones, lr, false);
      }
      // O^T += V^T P^T over the 16 keys (16x16x16 MFMA: V^T of dims 16d + c16,
      // keys 4 grp .. from one transposing read)
      const s16x4 bh_ = __builtin_bit_cast(s16x4, ph), bl_ = __builtin_bit_cast(s16x4, pl);
      const int rv = 16 * kb_w + 4 * grp + (c16 >> 2);
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        const s16x4 vop = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(vs + v_piece<DV>(rv, d, c16 & 3)));
        oacc[d][0] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, bh_, oacc[d][0], 0, 0, 0);
        oacc[d][0] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, bl_, oacc[d][0], 0, 0, 0);
      }
    };
    auto dstep = [&](int kt, const uint16_t* kc, const uint16_t* vc, uint16_t* kn,
                     uint16_t* vn) {
      // this thread's copies of tile kt have landed (those of the two tiles
      // after it may still be in flight: the counter drains in order), then
      // every thread's
      if (kt + 2 < n_kt)
        wait_vmem_n<2 * R>();
      else if (kt + 1 < n_kt)
        wait_vmem_n<R>();
      else
        wait_vmem();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (kt + 3 < n_kt) {
        issue_k(kt + 3, kn);
        issue_v(kt + 3, vn);
      }
      if (wave < 4) tile_work(kt, kc, vc);
    };
    for (int t0 = kt_first; t0 < n_kt; t0 += 4) {
      dstep(t0, k0s, v0s, k3s, v3s);
      if (t0 + 1 < n_kt) dstep(t0 + 1, k1s, v1s, k0s, v0s);
      if (t0 + 2 < n_kt) dstep(t0 + 2, k2s, v2s, k1s, v1s);
      if (t0 + 3 < n_kt) dstep(t0 + 3, k3s, v3s, k2s, v2s);
    }

    // ---- merge of the waves' states: each wave's O (f32, unnormalised) and
    // its max and sum per row go to LDS (two waves per K stage, the maxima
    // and sums in V stage 0), then every thread merges a few elements ----
    const float l_tot = group_sum(lr);
    wait_vmem();
    __syncthreads();
    {
      float* part = reinterpret_cast<float*>(wave < 2 ? k0s : wave < 4 ? k1s : wave < 6 ? k2s : k3s) +
                    (wave & 1) * 16 * DV;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
        *reinterpret_cast<f32x4*>(part + c16 * DV + 16 * d + 4 * grp) = oacc[d][0];
      float* ml = reinterpret_cast<float*>(v0s);
      if (grp == 0) {
        ml[wave * 16 + c16] = mu;
        ml[128 + wave * 16 + c16] = l_tot;
      }
    }
    __syncthreads();
    const float* ml = reinterpret_cast<const float*>(v0s);
    const float* parts[8] = {reinterpret_cast<const float*>(k0s),
                             reinterpret_cast<const float*>(k0s) + 16 * DV,
                             reinterpret_cast<const float*>(k1s),
                             reinterpret_cast<const float*>(k1s) + 16 * DV,
                             reinterpret_cast<const float*>(k2s),
                             reinterpret_cast<const float*>(k2s) + 16 * DV,
                             reinterpret_cast<const float*>(k3s),
                             reinterpret_cast<const float*>(k3s) + 16 * DV};
#pragma unroll
    for (int i = 0; i < 16 * DV / NT; ++i) {
      const int idx = tid + NT * i, r = idx / DV, dcol = idx % DV;
      if (q0 + r < ql) {
        float m = -FLT_MAX;
#pragma unroll
        for (int w = 0; w < 8; ++w) m = __builtin_fmaxf(m, ml[w * 16 + r]);
        float z = 0.0f, o = 0.0f;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const float sc = __builtin_amdgcn_exp2f(ml[w * 16 + r] - m);
          z += ml[128 + w * 16 + r] * sc;
          o += parts[w][r * DV + dcol] * sc;
        }
        const bool empty = !(z > 0.0f);
        const int64_t prow = ((int64_t)split * a.B * a.H + bh) * ql + q0 + r;
        a.ws_o[prow * DV + dcol] = empty ? 0.0f : o / z;
        if (dcol == 0) a.ws_l[prow] = empty ? -INFINITY : (m + __builtin_amdgcn_logf(z)) * kLn2;
      }
    }
    return false;
  } else if constexpr (NSTAGE == 4) {
    // copy instructions per thread per tile (K and V)
    constexpr int R = CopyShape<DK, BN, NT>::ROUNDS + CopyShape<DV, BN, NT>::ROUNDS;
    auto step4 = [&](int kt, const uint16_t* kc, const uint16_t* vc, uint16_t* kn,
                     uint16_t* vn) {
      // this thread's copies of tile kt have landed (the copies of the tiles
      // after it may still be in flight: the counter drains in order), then
      // every thread's
      if (kt + 2 < n_kt)
        wait_vmem_n<2 * R>();
      else if (kt + 1 < n_kt)
        wait_vmem_n<R>();
      else
        wait_vmem();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (kt + 3 < n_kt) {
        issue_k(kt + 3, kn);
        issue_v(kt + 3, vn);
      }
      if (kt >= wave_kt_first && kt < n_kw) {
        f32x4 s[NKB][kQB];
        scores(kc, s);
        if (kt >= mask_from) apply_mask(kt, s);
        float mx[kQB];
        if (__any(part_max(s, mx))) {
          complete_max(mx);
          rescale(mx, s);
        }
        bf16x8 phi[NKC][kQB], plo[NKC][kQB];
        probs(s, phi, plo);
        set_prio<2>();
        pv(vc, phi, plo);
        set_prio<0>();
      }
    };
    for (int kt = kt_first & ~3; kt < n_kt; kt += 4) {
      if (kt >= kt_first) step4(kt, k0s, v0s, k3s, v3s);
      if (kt + 1 >= kt_first && kt + 1 < n_kt) step4(kt + 1, k1s, v1s, k0s, v0s);
      if (kt + 2 >= kt_first && kt + 2 < n_kt) step4(kt + 2, k2s, v2s, k1s, v1s);
      if (kt + 3 >= kt_first && kt + 3 < n_kt) step4(kt + 3, k3s, v3s, k2s, v2s);
    }
  } else if constexpr (PAIRED) {
    for (int kt = kt_first & ~1; kt < n_kt; kt += 2) {
      if (kt >= kt_first) step(kt, k0s, v0s, k1s, v1s);
      if (kt + 1 < n_kt) step(kt + 1, k1s, v1s, k0s, v0s);
    }
  } else {
    for (int kt = kt_first; kt < n_kt; ++kt) {
      const bool odd = kt & 1;
      step(kt, odd ? k1s : k0s, odd ? v1s : v0s, odd ? k0s : k1s, odd ? v0s : v1s);
    }
  }

  // ---- epilogue: O = O_acc / l (+0 for an empty row), L = (m + log2 l) ln 2 ----
  float l_tot[kQB];
  bool write[kQB];
  bool wg_any = false;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int qrow = qw0 + 16 * qb + c16;
    const bool row_ok = compute && qrow < ql;
    l_tot[qb] = group_sum(l_run[qb]);
    write[qb] = REDO ? row_ok && redo[qb] : row_ok;
    if (!PRECISE) {
      // rows whose plain result is not accurate enough are redone compensated
      float omax = 0.0f;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) omax = __builtin_fmaxf(omax, __builtin_fabsf(oacc[d][qb][i]));
      omax = group_max(omax);
      redo[qb] = row_ok && l_tot[qb] > 0.0f && omax >= kRecheckO * l_tot[qb];
      write[qb] = row_ok && !redo[qb];
    }
  }
  if (!PRECISE) {
    // one flag per wave, then every wave reads all of them (every tile copy
    // has landed here: the last key step waited for its own)
    bool mine = false;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) mine |= redo[qb];
    const bool wave_any = __any(mine);
    if (lane == 0) wg_flags[wave] = wave_any;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < C::W; ++w) wg_any |= wg_flags[w] != 0;
  }
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int qrow = qw0 + 16 * qb + c16;
    if (write[qb]) {
      float lt = l_tot[qb], mu = m_use[qb], osc = 1.0f;
      if constexpr (!SPLIT) {
        // a sink logit of the row's head: one more term of the softmax with a
        // zero value, folded into the max and the sum here (an empty row then
        // gets O = 0 and L = the sink)
        if (a.sinks) {
          const int sh = a.sink_group > 1 ? h * a.sink_group + qrow : h;
          const float s2 = a.sinks[sh] * kLog2e;
          const float mf = __builtin_fmaxf(mu, s2);
          osc = __builtin_amdgcn_exp2f(mu - mf);
          lt = lt * osc + __builtin_amdgcn_exp2f(s2 - mf);
          mu = mf;
        }
      }
      const bool empty = !(lt > 0.0f);
      const float inv = empty ? 0.0f : __builtin_amdgcn_rcpf(lt) * osc;
      const float lse = empty ? -INFINITY : (mu + __builtin_amdgcn_logf(lt)) * kLn2;
      if constexpr (SPLIT) {
        // the chunk's partial: O normalised by its own sum (f32), and its L
        const int64_t prow = ((int64_t)split * a.B * a.H + bh) * ql + qrow;
        float* op = a.ws_o + prow * DV + 4 * grp;
#pragma unroll
        for (int d = 0; d < NDB; ++d) {
          f32x4 ov;
#pragma unroll
          for (int i = 0; i < 4; ++i) ov[i] = empty ? 0.0f : oacc[d][qb][i] * inv;
          *reinterpret_cast<f32x4*>(op + 16 * d) = ov;
        }
        if (grp == 0) a.ws_l[prow] = lse;
      } else {
        uint16_t* orow = a.o + b * a.o_sb + h * a.o_sh + (int64_t)qrow * a.o_sr + 4 * grp;
#pragma unroll
        for (int d = 0; d < NDB; ++d) {
          bf16x4 ov;
#pragma unroll
          for (int i = 0; i < 4; ++i) ov[i] = empty ? (__bf16)0.0f : (__bf16)(oacc[d][qb][i] * inv);
          *reinterpret_cast<bf16x4*>(orow + 16 * d) = ov;
        }
        if (grp == 0) lrow_base[qrow] = lse;
      }
    }
  }
  // no LDS copy may still be in flight when the workgroup ends (waiting for
  // the stores here too was measured faster for D=256 than leaving them)
  wait_vmem();
  return wg_any;
}

template <int DK, int DV, bool CAUSAL, bool WINDOW, int MASK, int MODE, int QBX = 0>
__global__ __launch_bounds__((64 * KCfg<DK, DV, WINDOW>::W))
__attribute__((amdgpu_waves_per_eu(MODE == kMixed ? KCfg<DK, DV, WINDOW>::WPE : 2))) void fa_fwd_kernel(
    FwdArgs a) {
  static_assert(MODE < kSplit || (MASK == kNoMask && !WINDOW),
                "split-KV and paged: unmasked, no window");
  static_assert(MODE != kMixed || MASK == kNoMask, "the masked forward always runs compensated");
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using C = KCfg<DK, DV, WINDOW>;
  constexpr int TILE_K = C::BN * DK, TILE_V = C::BN * DV;
  __shared__ __attribute__((aligned(1024))) uint16_t k0s[TILE_K];
  __shared__ __attribute__((aligned(1024))) uint16_t v0s[TILE_V];
  __shared__ __attribute__((aligned(1024))) uint16_t k1s[TILE_K];
  __shared__ __attribute__((aligned(1024))) uint16_t v1s[TILE_V];
  // (the third and fourth stages of the split-KV and paged pipelines)
  constexpr int TILE_X = MODE >= kSplit && DK <= 128 ? TILE_K : 8;
  __shared__ __attribute__((aligned(1024))) uint16_t k2s[TILE_X];
  __shared__ __attribute__((aligned(1024))) uint16_t v2s[TILE_X];
  __shared__ __attribute__((aligned(1024))) uint16_t k3s[TILE_X];
  __shared__ __attribute__((aligned(1024))) uint16_t v3s[TILE_X];
  __shared__ int wg_flags[C::W];

  // ---- work item ----
  // Workgroups are handed to the 8 XCDs round-robin (bid mod 8). When B*H is a
  // multiple of 8, XCD x owns the heads [x*per, (x+1)*per) (so one KV group
  // stays within one XCD's L2), takes them in groups of 8 (when per is a
  // multiple of 8; fewer K/V in flight per L2) and walks each group's query
  // tiles heaviest (most keys) first, so the cheap tiles fill the tail.
  // (Groups of 1, 2 or 4 heads were measured slower, 8 faster than all.)
  // (split-KV: the chunk index is the fastest-varying part of the block index)
  const int BH = a.B * a.H;
  constexpr bool SPLIT_GRID = MODE == kSplit || MODE == kPagedSplit || MODE == kPagedBlocksSplit;
  const int split = SPLIT_GRID ? (int)(blockIdx.x % (unsigned)a.n_split) : 0;
  const int bid = SPLIT_GRID ? (int)(blockIdx.x / (unsigned)a.n_split) : (int)blockIdx.x;
  int qt_rev, bh;
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, tl = bid >> 3, per = BH >> 3;
    const int gh = (per & 7) == 0 ? 8 : per;  // heads per group
    const int gsz = gh * a.qt_count;          // workgroups per group
    const int gi = tl / gsz, r = tl % gsz;
    qt_rev = r / gh;
    bh = xcd * per + gi * gh + r % gh;
  } else {
    qt_rev = bid / BH;
    bh = bid % BH;
  }
  const int qtile = a.qt_base + a.qt_count - 1 - qt_rev;
  bool redo[C::QB] = {};
#define FA_TILE_BUFFERS k0s, v0s, k1s, v1s, k2s, v2s, k3s, v3s
  if constexpr (MODE == kMixed) {
    // the compensated tiles are the lightest, so they run last and fill the tail
    if (qtile < a.n_precise) {
      fwd_tile<DK, DV, CAUSAL, WINDOW, kNoMask, true, false>(a, qtile, bh, FA_TILE_BUFFERS, redo,
                                                             wg_flags);
    } else if (fwd_tile<DK, DV, CAUSAL, WINDOW, kNoMask, false, false>(
                   a, qtile, bh, FA_TILE_BUFFERS, redo, wg_flags)) {
      // (the plain pass's last barrier came after every wave's last LDS read,
      // so the redo's copies may reuse the tile buffers)
      fwd_tile<DK, DV, CAUSAL, WINDOW, kNoMask, true, true>(a, qtile, bh, FA_TILE_BUFFERS, redo,
                                                            wg_flags);
    }
  } else if constexpr (MODE >= kSplit && MODE <= kPagedBlocksSplit) {
    // Split-KV and paged: a chunk of a query tile (unsplit paged: the
    // sequence's whole key range) runs compensated when some of its rows see 1
    // to kPreciseKeys - 1 of its keys (by position, as the mixed kernel's short
    // tiles), when the problem (a paged sequence) has at most kPlainMinKeys
    // keys, or when plain tiles are off for the call; otherwise plain, with the
    // compensated redo of rows with some |O| >= 1. The decoding kernels (QBX)
    // stay compensated.
    constexpr bool SP = SPLIT_GRID;
    constexpr bool PG = MODE != kSplit;
    constexpr bool SB = MODE == kPagedBlocks || MODE == kPagedBlocksSplit;
    bool precise = true;
    if constexpr (QBX == 0) {
      // (paged: the sequence's own key count and causal offset, as fwd_tile
      // takes them)
      const int kl = PG ? min(max(load_uniform(a.seq_lens, bh / a.H), 0),
                              a.max_blocks * a.block_size)
                        : a.kl;
      const int off = PG ? max(kl - a.ql, 0) : a.causal_off;
      const int c0 = SP ? split * a.kchunk : 0, c1 = SP ? min(c0 + a.kchunk, kl) : kl;
      constexpr int kBM = block_m<DK, DV>();
      const int r0 = qtile * kBM, r1 = min(r0 + kBM, a.ql) - 1;
      const int n_first = max(0, (CAUSAL ? min(c1, off + r0 + 1) : c1) - c0);
      const int n_last = max(0, (CAUSAL ? min(c1, off + r1 + 1) : c1) - c0);
      precise = !a.split_plain || (PG && kl <= kPlainMinKeys) ||
                (n_first < kPreciseKeys && n_last >= 1);
    }
    if (precise) {
      fwd_tile<DK, DV, CAUSAL, false, kNoMask, true, false, SP, PG, SB, QBX>(
          a, qtile, bh, FA_TILE_BUFFERS, redo, wg_flags, split);
    } else if constexpr (QBX == 0) {
      if (fwd_tile<DK, DV, CAUSAL, false, kNoMask, false, false, SP, PG, SB>(
              a, qtile, bh, FA_TILE_BUFFERS, redo, wg_flags, split))
        fwd_tile<DK, DV, CAUSAL, false, kNoMask, true, true, SP, PG, SB>(
            a, qtile, bh, FA_TILE_BUFFERS, redo, wg_flags, split);
    }
  } else {
    fwd_tile<DK, DV, CAUSAL, WINDOW, MASK, true, false>(a, qtile, bh, FA_TILE_BUFFERS, redo,
                                                        wg_flags);
  }
#undef FA_TILE_BUFFERS
#endif
}

// Merge of the split-KV partials of each row (one wave per row, lane l holds
// dims l*P .. l*P+P-1): L = m + ln sum_s exp(L_s - m), O = sum_s exp(L_s - L) O_s,
// the same merge through L that combines key partitions computed apart.
struct CombineArgs {
  const float* ws_o;  // [n_split, rows, D]
  const float* ws_l;  // [n_split, rows]
  uint16_t* o;        // bf16 [rows, D]
  float* l;           // f32 [rows]
  int64_t rows;       // B * H * ql
  int n_split;
  int H, ql;
  int64_t o_sb, o_sh;  // O's element strides of batch, head and row
  int o_sr;
  const float* sinks;  // sink logits as in FwdArgs (null: none), merged once here
  int sink_group;
};

template <int D>
__global__ __launch_bounds__(256) void fa_combine_kernel(CombineArgs c) {
  // One workgroup per row: the four waves read the chunks' partials in
  // parallel (wave w the chunks s = w mod 4, several loads in flight each),
  // then their sums are added through LDS. (A serial walk over the chunks,
  // one load latency per chunk, took longer than the partials themselves.)
  constexpr int P = D / 64;
  __shared__ float red_o[4][D];
  __shared__ float red_z[4], red_m[4];
  const int64_t row = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // the largest chunk logsumexp of the row
  float m = -INFINITY;
  for (int s = threadIdx.x; s < c.n_split; s += 256) m = fmaxf(m, c.ws_l[s * c.rows + row]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) red_m[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
  // the row's sink: one more term of the merged sum with a zero value
  const int64_t bh = row / c.ql;
  float sink = -INFINITY;
  if (c.sinks) {
    const int h = (int)(bh % c.H);
    sink = c.sinks[c.sink_group > 1 ? h * c.sink_group + (int)(row % c.ql) : h];
    m = fmaxf(m, sink);
  }
  float acc[P] = {};
  float z = 0.0f;
  if (m != -INFINITY) {
#pragma unroll 8
    for (int s = wave; s < c.n_split; s += 4) {
      // (a chunk with no visible key has L_s = -inf: weight 0, partial O 0)
      const float w = __builtin_amdgcn_exp2f((c.ws_l[s * c.rows + row] - m) * kLog2e);
      z += w;
      const float* op = c.ws_o + (s * c.rows + row) * D + lane * P;
#pragma unroll
      for (int e = 0; e < P; ++e) acc[e] += w * op[e];
    }
  }
#pragma unroll
  for (int e = 0; e < P; ++e) red_o[wave][lane * P + e] = acc[e];
  if (lane == 0) red_z[wave] = z;
  __syncthreads();
  if (wave != 0) return;
  z = (red_z[0] + red_z[1]) + (red_z[2] + red_z[3]);
  const bool empty = m == -INFINITY;
  if (!empty) z += __builtin_amdgcn_exp2f((sink - m) * kLog2e);
  const float inv = empty ? 0.0f : 1.0f / z;
  uint16_t* orow = c.o + (bh / c.H) * c.o_sb + (bh % c.H) * c.o_sh + (row % c.ql) * c.o_sr +
                   lane * P;
#pragma unroll
  for (int e = 0; e < P; ++e) {
    const int d = lane * P + e;
    const float o = (red_o[0][d] + red_o[1][d]) + (red_o[2][d] + red_o[3][d]);
    orow[e] = __builtin_bit_cast(uint16_t, empty ? (__bf16)0.0f : (__bf16)(o * inv));
  }
  if (lane == 0) c.l[row] = empty ? -INFINITY : m + __builtin_amdgcn_logf(z) * kLn2;
}

template <int DK, int DV, bool CAUSAL, bool WINDOW, int MASK, int MODE, int QBX = 0>
hipError_t launch(const FwdArgs& a, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_kernel<DK, DV, CAUSAL, WINDOW, MASK, MODE, QBX>), dim3(grid),
                     dim3(64 * KCfg<DK, DV, WINDOW>::W), 0, stream, a);
  return hipGetLastError();
}

// Masked: one compensated launch over all query tiles. Unmasked: the mixed
// launch over all tiles (compensated for the tiles with short rows, the first
// n_short ones; plain for the others, with a compensated redo of the rows
// that need it inside the same workgroup).
template <int DK, int DV, bool CAUSAL, bool WINDOW>
hipError_t dispatch_c(FwdArgs a, int mask, int n_short, hipStream_t stream) {
  const unsigned bh = (unsigned)(a.B * a.H);
  const int n_qt = a.n_qtiles;
  a.qt_base = 0;
  a.qt_count = n_qt;
  if (mask != kNoMask) {
    a.n_precise = n_qt;
    const unsigned grid = bh * n_qt;
    return mask == kMaskBF16   ? launch<DK, DV, CAUSAL, WINDOW, kMaskBF16, kAll>(a, grid, stream)
           : mask == kMaskBool ? launch<DK, DV, CAUSAL, WINDOW, kMaskBool, kAll>(a, grid, stream)
                               : launch<DK, DV, CAUSAL, WINDOW, kMaskF32, kAll>(a, grid, stream);
  }
  a.n_precise = n_short;
  return launch<DK, DV, CAUSAL, WINDOW, kNoMask, kMixed>(a, bh * n_qt, stream);
}

// Split-KV: the partials over all (chunk, head, query tile), then the merge.
// (MODE: kSplit, kPagedSplit or kPagedBlocksSplit)
template <int DK, int DV, bool CAUSAL, int MODE = kSplit>
hipError_t dispatch_split(FwdArgs a, hipStream_t stream) {
  const unsigned bh = (unsigned)(a.B * a.H);
  a.qt_base = 0;
  a.qt_count = a.n_qtiles;
  a.n_precise = a.n_qtiles;
  // (at most 16 query rows: the narrow kernel, one 16-row block per wave,
  // where the pair's waves hold two)
  const unsigned grid = bh * (unsigned)a.n_qtiles * (unsigned)a.n_split;
  hipError_t e;
  if constexpr (Cfg<DK, DV>::QB > 1)
    e = a.ql <= 16 ? launch<DK, DV, CAUSAL, false, kNoMask, MODE, 1>(a, grid, stream)
                   : launch<DK, DV, CAUSAL, false, kNoMask, MODE>(a, grid, stream);
  else
    e = launch<DK, DV, CAUSAL, false, kNoMask, MODE>(a, grid, stream);
  if (e != hipSuccess) return e;
  CombineArgs c;
  c.ws_o = a.ws_o;
  c.ws_l = a.ws_l;
  c.o = a.o;
  c.l = a.l;
  c.rows = (int64_t)a.B * a.H * a.ql;
  c.n_split = a.n_split;
  c.H = a.H;
  c.ql = a.ql;
  c.o_sb = a.o_sb;
  c.o_sh = a.o_sh;
  c.o_sr = a.o_sr;
  c.sinks = a.sinks;
  c.sink_group = a.sink_group;
  hipLaunchKernelGGL(fa_combine_kernel<DV>, dim3((unsigned)c.rows), dim3(256), 0, stream, c);
  return hipGetLastError();
}

// Paged KV: one compensated launch over all query tiles, or the split-KV pair.
template <int D, int MODE, int SPLIT_MODE>
hipError_t dispatch_paged_m(FwdArgs a, bool causal, hipStream_t stream) {
  if (a.n_split > 0)
    return causal ? dispatch_split<D, D, true, SPLIT_MODE>(a, stream)
                  : dispatch_split<D, D, false, SPLIT_MODE>(a, stream);
  const unsigned grid = (unsigned)(a.B * a.H) * (unsigned)a.n_qtiles;
  a.qt_base = 0;
  a.qt_count = a.n_qtiles;
  a.n_precise = a.n_qtiles;
  return causal ? launch<D, D, true, false, kNoMask, MODE>(a, grid, stream)
                : launch<D, D, false, false, kNoMask, MODE>(a, grid, stream);
}

template <int D>
hipError_t dispatch_paged(const FwdArgs& a, bool causal, hipStream_t stream) {
  return a.block_size % Cfg<D, D>::BN == 0
             ? dispatch_paged_m<D, kPaged, kPagedSplit>(a, causal, stream)
             : dispatch_paged_m<D, kPagedBlocks, kPagedBlocksSplit>(a, causal, stream);
}

// One (DK, DV) pair: split-KV (64, 128 and 256 only), or the sliding-window,
// causal or full forward.
template <int DK, int DV>
hipError_t dispatch_d(const FwdArgs& a, bool causal, bool window, int mask, int n_short,
                      hipStream_t stream) {
  if constexpr (DK == DV && !kPanels<DK>) {
    if (a.n_split > 0)
      return causal ? dispatch_split<DK, DV, true>(a, stream)
                    : dispatch_split<DK, DV, false>(a, stream);
  } else if (a.n_split > 0) {
    return hipErrorInvalidValue;
  }
  if (window) return dispatch_c<DK, DV, true, true>(a, mask, n_short, stream);
  return causal ? dispatch_c<DK, DV, true, false>(a, mask, n_short, stream)
                : dispatch_c<DK, DV, false, false>(a, mask, n_short, stream);
}

}  // namespace
