// fa_bwd.hip - flash-attention training backward (dQ, dK, dV) for AMD MI355X
// (gfx950).
//
// What is computed is the FA-2 backward of the method's page ("mlx-native
// 0.9.0", tests/test_flash_attn_train.rs, section "Phase 2 - backward kernel
// helpers", the CPU oracle sdpa_backward_reference_f32), with the forward's
// causal alignment (key j hidden from query row i when j > max(kl - ql, 0) + i):
//
//   S_ij  = scale * q_i . k_j (+ mask_ij)       P_ij = exp(S_ij - L_i)
//   dP_ij = dO_i . v_j                          D_i  = sum_d O_id dO_id
//   dS_ij = P_ij (dP_ij - D_i)
//   dQ_i  = scale * sum_j dS_ij k_j             dK_j = scale * sum_i dS_ij q_i
//   dV_j  = sum_i P_ij dO_i                     (dK, dV summed over a GQA group)
//
// (D_i = rowsum(dO_i * O_i) equals the page's sum_j P_ij dP_ij when O is the
// forward's output.) The WINDOW variants apply the forward's sliding window
// (key j visible to row i iff q_abs - window <= j <= q_abs) and stream only the
// tiles inside the band. Three launches (four with sinks), no atomics and no
// workspace:
//
//   rows pass:         per query row, L2_i = L_i log2(e) (+inf for a row with
//                      no visible key) and -D_i, stored as two floats at the
//                      start of the row's dQ memory (dQ is written only by the
//                      last launch, so until then its rows serve as scratch)
//   dKV pass (kBwdKV): fixed = key rows (K, V), streamed = query rows of every
//                      head of the group (Q, dO, and L2, -D per row)
//   dQ pass  (kBwdQ):  fixed = query rows (Q, dO, and their L2, -D, read
//                      before the rows are overwritten), streamed = keys (K, V)
//
// With attention sinks the rows pass also stores each row's term of its
// head's sink gradient, which one more launch sums per head before the dQ
// pass (fa_bwd_sinks_kernel).
//
// The last two share one kernel template: a workgroup keeps a block of "fixed"
// rows in registers and streams tiles of the other side through LDS.
// Per streamed tile every wave computes, with v_mfma_f32_16x16x32_bf16 and the
// same operand layouts as the forward kernel,
//   S^T  = Y1 X1^T (raw scores)   dP^T = Y2 X2^T
// (Y1/Y2 = streamed K/V or Q/dO rows read from LDS as the A operand, rows
// permuted by key_of so that the products' C layout is the next product's B
// layout; X1/X2 = fixed Q/dO or K/V rows held as the B operand), then P and dS
// element by element, and
//   dQ pass:  dQ^T += Y1^T dS^T
//   dKV pass: dK^T += Y1^T dS,  dV^T += Y2^T P
// with Y1^T, Y2^T read from the LDS tiles by ds_read_b64_tr_b16. P and dS
// enter the MFMAs rounded to bf16; the sums are f32.
#include <hip/hip_runtime.h>

#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "fa.h"
#include "fa_common.h"

namespace {

constexpr int kBwdQ = 0, kBwdKV = 1;

// Per head dim and pass: W waves, FB fixed 16-row blocks per wave, BN streamed
// rows per tile, WPE waves per SIMD (register budget).
template <int D, int PASS> struct BwdCfg;
// DS waves may share each fixed block, each accumulating D/DS of the output
// dims (both then compute the block's full S and dP); every pass now runs
// DS = 1. With the operand reads' XOR addressing the D=256 dK/dV pass holds
// one 16-key block with its full dK and dV per wave at two waves per SIMD
// (240 VGPRs; two waves per block: 4.96 -> 3.99 ms for D=256 GQA 8k causal),
// and the D=64 dK/dV pass one block per wave at four waves per SIMD, streaming
// 128-row tiles (2% faster than 64 for D=64; slower for D=128). The D=64
// dQ pass keeps one 16-row block per wave at four waves per SIMD (two
// workgroups per CU).
template <> struct BwdCfg<64, kBwdQ> { static constexpr int W = 8, FB = 1, BN = 64, WPE = 4, DS = 1; };
template <> struct BwdCfg<64, kBwdKV> { static constexpr int W = 8, FB = 1, BN = 128, WPE = 4, DS = 1; };
template <> struct BwdCfg<128, kBwdQ> { static constexpr int W = 8, FB = 1, BN = 64, WPE = 2, DS = 1; };
template <> struct BwdCfg<128, kBwdKV> { static constexpr int W = 8, FB = 1, BN = 64, WPE = 2, DS = 1; };
template <> struct BwdCfg<256, kBwdQ> { static constexpr int W = 8, FB = 1, BN = 64, WPE = 2, DS = 1; };
template <> struct BwdCfg<256, kBwdKV> { static constexpr int W = 8, FB = 1, BN = 32, WPE = 2, DS = 1; };
template <int D, int PASS> constexpr int fixed_rows() {
  return BwdCfg<D, PASS>::W / BwdCfg<D, PASS>::DS * 16 * BwdCfg<D, PASS>::FB;
}

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dO;
  const float* L;            // rows pass only (the others read L2 from dQ's rows)
  const void* mask;          // f32, bf16 or bool bytes (the kernel's MASK), or null
  int64_t mask_sb, mask_sh;  // mask strides of batch and head, in elements (0: broadcast)
  int mask_sr;               // mask row stride, in elements (kl: rows contiguous)
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int B, H, Hkv, ql, kl;
  int group;         // H / Hkv
  int n_ftiles;      // fixed-row tiles per (batch, head) of the fixed side
  int causal_off;    // max(kl - ql, 0)
  int window;        // WINDOW variants: keys below q_abs - window are hidden
  float scale;       // signed softmax scale (multiplies dQ and dK)
  float c;           // scale * log2(e), never 0 (exp2 argument factor)
  // element strides of batch, head and row (head_dim contiguous): q_* for Q,
  // O, dO and dQ, k_* for K, V, dK and dV; L is contiguous [B, H, ql]
  int64_t q_sb, q_sh, k_sb, k_sh;
  int q_sr, k_sr;
  const float* sinks;  // per-head sink logits [H] (natural log), or null
  float* dsinks;       // their gradient [H] (written when sinks is set)
};

// x ^ c computed in the iteration that uses it: an asm that also takes the
// loop's tile index (unused), so the compiler can neither hoist it out of the
// loop nor fold it, and one base offset stays live in place of one register
// per XOR pattern (c wave-uniform). Not volatile: it schedules as an ordinary
// VALU instruction (a volatile asm held the LDS reads in place, 4-15% slower).
__device__ __forceinline__ int xor_here(int x, int c, int t) {
  int r;
  asm("v_xor_b32 %0, %1, %2 ; tile %3" : "=v"(r) : "s"(c), "v"(x), "s"(t));
  return r;
}

template <bool B> struct BoolTag { static constexpr bool value = B; };

// log2-units logsumexp of a row; a row with no visible key (L = -inf) gets
// +inf, so that every P of that row is 0
__device__ __forceinline__ float lse2(float l) { return l == -INFINITY ? INFINITY : l * kLog2e; }

// The rows pass: for every query row, (L2, -D) = (lse2(L), -sum_d O_d dO_d) as
// two floats at the start of the row's dQ memory (8 of its >= 128 bytes, 16
// with sinks; dQ's rows are 16-byte aligned). D/8 lanes per row, 16 bytes of
// O and dO each; a grid-stride loop over groups of 256/(D/8) rows.
template <int D>
__global__ __launch_bounds__(256) void fa_bwd_rows_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  const int part = threadIdx.x % LPR;
  const int64_t nrows = (int64_t)a.B * a.H * a.ql;
  for (int64_t r0 = (int64_t)blockIdx.x * RPB; r0 < nrows; r0 += (int64_t)gridDim.x * RPB) {
    const int64_t row = r0 + threadIdx.x / LPR;
    const bool live = row < nrows;
    int64_t base = 0;
    float acc = 0.0f;
    if (live) {
      const int64_t bh = row / a.ql;
      const int i = (int)(row - bh * a.ql);
      base = bh / a.H * a.q_sb + bh % a.H * a.q_sh + (int64_t)i * a.q_sr;
      const bf16x8 ov = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(a.o + base + 8 * part));
      const bf16x8 gv = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(a.dO + base + 8 * part));
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += (float)ov[e] * (float)gv[e];
    }
    // (LPR divides 64: a row's lanes are consecutive lanes of one wave)
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m, 64);
    if (live && part == 0) {
      const float l2 = lse2(a.L[row]);
      if (a.sinks) {
        // with sinks, also the row's term of its head's sink gradient,
        // p (-D) with p = exp(sink - L) the sink's weight (0 for a -inf
        // sink), as a third float of the row
        const float p = __builtin_amdgcn_exp2f(a.sinks[row / a.ql % a.H] * kLog2e - l2);
        *reinterpret_cast<float4*>(a.dq + base) = make_float4(l2, -acc, p * -acc, 0.0f);
      } else {
        *reinterpret_cast<float2*>(a.dq + base) = make_float2(l2, -acc);
      }
    }
  }
}

// The sink gradient of head blockIdx.x: the sum, over every batch and row,
// of the rows pass's third float, in a fixed order (each thread a strided
// run of the rows, then a tree over the threads), so the result is
// deterministic. It runs before the dQ pass overwrites the rows.
__global__ __launch_bounds__(256) void fa_bwd_sinks_kernel(BwdArgs a) {
  __shared__ float part[256];
  const int h = blockIdx.x;
  const int64_t n = (int64_t)a.B * a.ql;
  float acc = 0.0f;
  for (int64_t t = threadIdx.x; t < n; t += 256) {
    const int64_t b = t / a.ql, i = t - b * a.ql;
    acc += reinterpret_cast<const float*>(a.dq + b * a.q_sb + h * a.q_sh + i * a.q_sr)[2];
  }
  part[threadIdx.x] = acc;
  __syncthreads();
#pragma unroll
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.dsinks[h] = part[0];
}

template <int D, int PASS, bool CAUSAL, bool WINDOW, int MASK>
__global__ __launch_bounds__((64 * BwdCfg<D, PASS>::W))
__attribute__((amdgpu_waves_per_eu(BwdCfg<D, PASS>::WPE))) void fa_bwd_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using C = BwdCfg<D, PASS>;
  constexpr int BN = C::BN;
  constexpr int FB = C::FB;
  constexpr int FR = fixed_rows<D, PASS>();
  constexpr int NKB = BN / 16;  // 16-row blocks of a streamed tile
  constexpr int NKC = BN / 32;  // 32-row chunks (contraction steps of the second products)
  static_assert(BN == 32 || BN == 64 || BN == 128, "a tile is 1, 2 or 4 chunks of 32 rows");
  constexpr int NRW = BN > 64 ? BN / 64 : 1;  // waves that copy the tile's (L2, D) rows
  constexpr int NDB = D / 16;   // 16-dim blocks
  constexpr int DS = C::DS;
  constexpr int NDA = NDB / DS;  // 16-dim blocks of this wave's accumulators
  static_assert(NDA * DS == NDB && C::W % DS == 0, "dims split evenly");
  constexpr int NDS = D / 32;   // 32-dim steps
  constexpr int TILE = BN * D;
  constexpr int NT = 64 * C::W;
  constexpr bool KV = PASS == kBwdKV;
  constexpr bool HAS_MASK = MASK != kNoMask;
  static_assert(CAUSAL || !WINDOW, "the sliding window includes the causal rule");
  // the two stages of each streamed operand are separate arrays, so that the
  // compiler can tell a stage's reads from the copy into the other one
  __shared__ __attribute__((aligned(1024))) uint16_t y1s0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t y1s1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t y2s0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t y2s1[TILE];
  // dKV pass: L2 and D of the streamed rows (the first 16 bytes of their dQ
  // rows: L2, D and two unused floats), one array per stage, copied with the
  // stage's tiles (64 entries: one per lane of the copying wave)
  __shared__ float4 srow0[KV ? 64 * NRW : 1];
  __shared__ float4 srow1[KV ? 64 * NRW : 1];

  const int tid = threadIdx.x;
  // wave-uniform wave index: every wave-level condition is a scalar branch
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int c16 = lane & 15;
  const int grp = lane >> 4;

  // ---- work item: heaviest first under causal masking ----
  // dQ pass: late query tiles see the most keys; dKV pass: early key tiles are
  // seen by the most queries.
  const int nfh = KV ? a.B * a.Hkv : a.B * a.H;  // fixed (batch, head) pairs
  const int bid = blockIdx.x;
  const int fhead = bid % nfh;
  const int ftile = KV ? bid / nfh : a.n_ftiles - 1 - bid / nfh;
  const int b = fhead / (KV ? a.Hkv : a.H);
  const int hf = fhead % (KV ? a.Hkv : a.H);     // fixed head (query head or kv head)
  const int g = KV ? hf : hf / a.group;           // kv head
  const int ql = a.ql, kl = a.kl, off = a.causal_off;
  const int nfixed = KV ? kl : ql;
  const int nstream = KV ? ql : kl;
  const int f0 = ftile * FR;
  const int dpart = wave / (C::W / DS);  // this wave's part of the output dims
  const int fw0 = f0 + (wave % (C::W / DS)) * 16 * FB;  // this wave's first fixed row
  const bool wave_active = fw0 < nfixed;

  const int64_t kv_base = b * a.k_sb + g * a.k_sh;
  const int64_t qh_base = b * a.q_sb + hf * a.q_sh;  // dQ pass: the fixed query head
  const uint16_t* x1p = KV ? a.k + kv_base : a.q + qh_base;
  const uint16_t* x2p = KV ? a.v + kv_base : a.dO + qh_base;
  const int xr = KV ? a.k_sr : a.q_sr;  // row strides of the fixed and streamed rows
  const int yr = KV ? a.q_sr : a.k_sr;

  // ---- fixed rows as B operands: block fb, step s: row fw0+16fb+c16, dims 32s+8grp.. ----
  bf16x8 x1op[FB][NDS], x2op[FB][NDS];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb) {
    const int r = min(fw0 + 16 * fb + c16, nfixed - 1);
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
      x1op[fb][s] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(x1p + (int64_t)r * xr + 32 * s + 8 * grp));
      x2op[fb][s] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(x2p + (int64_t)r * xr + 32 * s + 8 * grp));
    }
  }
  // dQ pass: L2 and -D of the fixed rows, from the rows pass (read here, before
  // this workgroup overwrites its rows; a wave past the end reads the last row,
  // whose values it never uses)
  float l2f[FB], dfx[FB];
  if constexpr (!KV) {
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
      const int r = min(fw0 + 16 * fb + c16, nfixed - 1);
      const float2 sv = *reinterpret_cast<const float2*>(a.dq + qh_base + (int64_t)r * a.q_sr);
      l2f[fb] = sv.x;
      dfx[fb] = sv.y;
    }
  }

  // ---- accumulators: dQ^T, or dK^T and dV^T (dims x fixed rows) ----
  f32x4 acc1[NDA][FB], acc2[NDA][FB];
#pragma unroll
  for (int d = 0; d < NDA; ++d)
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
      acc1[d][fb] = f32x4{};
      acc2[d][fb] = f32x4{};
    }

  // ---- streamed range ----
  // dQ pass: keys 0 .. kend of kv head g (under a window, from the first key the
  // workgroup's first row sees). dKV pass: for every query head of the group,
  // the query tiles from the first one that sees the workgroup's first key
  // (under a window, up to the last one that still sees its last key).
  const int flast = min(f0 + FR, nfixed) - 1;
  int n_per = 0, st_lo = 0;
  if constexpr (!KV) {
    const int kend = CAUSAL ? min(kl, off + flast + 1) : kl;
    st_lo = WINDOW ? max(0, off + f0 - a.window) / BN : 0;
    n_per = kend > 0 ? max(0, (kend + BN - 1) / BN - st_lo) : 0;
  } else {
    const int n_qt = (ql + BN - 1) / BN;
    st_lo = CAUSAL ? max(0, f0 - off) / BN : 0;
    const int q_last = flast - off + (WINDOW ? a.window : 0);  // last query seeing key flast
    const int st_hi = !WINDOW ? n_qt : q_last < 0 ? 0 : min(n_qt, q_last / BN + 1);
    n_per = max(0, st_hi - st_lo);
  }
  const int n_st = KV ? a.group * n_per : n_per;
  auto tile_head = [&](int t) { return KV ? g * a.group + t / n_per : hf; };
  auto tile_first = [&](int t) { return (st_lo + (KV ? t % n_per : t)) * BN; };
  auto y1_src = [&](int t) -> const uint16_t* {
    return KV ? a.q + b * a.q_sb + tile_head(t) * a.q_sh : a.k + kv_base;
  };
  auto y2_src = [&](int t) -> const uint16_t* {
    return KV ? a.dO + b * a.q_sb + tile_head(t) * a.q_sh : a.v + kv_base;
  };

  int y1off[CopyShape<D, BN, NT>::ROUNDS], y2off[CopyShape<D, BN, NT>::ROUNDS];
  copy_offsets<D, BN, NT, true>(tid, y1off, yr);
  copy_offsets<D, BN, NT, false>(tid, y2off, yr);
  auto issue = [&](int t, uint16_t* y1d, uint16_t* y2d) {
    issue_tile<D, BN, NT, true>(y1_src(t), tile_first(t), nstream, y1d, tid, 64 * wave, y1off,
                                yr);
    issue_tile<D, BN, NT, false>(y2_src(t), tile_first(t), nstream, y2d, tid, 64 * wave, y2off,
                                 yr);
  };
  // dKV pass: the first BN/64 waves (at least one) copy (L2, D) of tile t's
  // rows from the rows pass straight into LDS, one row per lane (rows past ql
  // repeat the last one),
  // with the same direct-to-LDS loads as the tiles (no registers held)
  auto issue_rows = [&](int t, float4* srow) {
    if (KV && wave < NRW) {
      const int first = tile_first(t);
      const int n = min(ql - first, BN);
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.dq + b * a.q_sb + tile_head(t) * a.q_sh + (int64_t)first * a.q_sr), 0,
          ((n - 1) * a.q_sr + 8) * 2, kRsrcWord3);
      // (the lane index recomputed here, in an asm the compiler cannot hoist:
      // kept live across the loop it was spilled, and its reload waited for
      // the tile copies in flight)
      int l;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(srow + 64 * wave), 16,
                                               min(64 * wave + l, n - 1) * a.q_sr * 2, 0, 0, 0);
    }
  };

  // ---- operand reads from the LDS tiles ----
  // Byte offsets in a tile of this lane's reads for s = 0, kb = 0 (row reads)
  // and d = 0, j = 0, t = 0 (transposed reads), per swizzle (K-type for Y1,
  // V-type for Y2). Row r's 16-byte chunk c sits at 2rD + 16 (c ^ sw(r)), and
  // the rows a lane reads for other kb, j and t differ from these by 4 or 32
  // rows, which leave sw unchanged; a row is a multiple of 128 bytes and the
  // chunk index below D/8, so the other reads are these offsets XORed with
  // 64 s (row reads: chunk 4s + grp) or 32 d (transposed: chunk 2d + (c16&3)/2),
  // plus whole rows.
  const int rr0 = key_of(0, c16);
  const int tr0 = 8 * grp + (c16 >> 2), tx = (c16 & 3) >> 1;
  const int rbase[2] = {2 * rr0 * D + 16 * (grp ^ kswz<D>(rr0)),
                        2 * rr0 * D + 16 * (grp ^ vswz<D>(rr0))};
  const int tbase[2] = {2 * tr0 * D + 16 * (tx ^ kswz<D>(tr0)) + 8 * (c16 & 1),
                        2 * tr0 * D + 16 * (tx ^ vswz<D>(tr0)) + 8 * (c16 & 1)};
  // row read (A operand of S^T / dP^T): streamed row key_of(kb, c16), dims 32s + 8grp..
  auto rread = [&](const uint16_t* buf, bool is_y1, int s, int kb, int t) {
    const int x = rbase[is_y1 ? 0 : 1];
    const int o = (s == 0 ? x : xor_here(x, 64 * s, t)) + 2 * D * (32 * (kb >> 1) + 4 * (kb & 1));
    // (one offset from the tile: a short address chain from the buffer, so
    // that the compiler keeps the buffer's alias scope on the read)
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(buf) + o);
  };
  // transposed read (A operand of the second products): dims 16d + c16, streamed
  // rows 32j + 8grp + (0..7)
  auto tread = [&](const uint16_t* buf, bool is_y1, int d, int j, int t) {
    const int x = tbase[is_y1 ? 0 : 1];
    const int o = xor_here(x, 32 * d, t) + 2 * D * 32 * j;
    s16x4 half[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const char* addr = reinterpret_cast<const char*>(buf) + (o + 2 * D * 4 * u);
      half[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)addr);
    }
    return __builtin_bit_cast(bf16x8,
                              __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // the two 16-row blocks (2j, 2j + 1) of 32-row chunk j of the streamed tile
  // (out enters holding the accumulators' starting values)
  auto products = [&](const uint16_t* buf, bool is_y1, const bf16x8 (&xop)[FB][NDS], int j,
                      int t, f32x4 (&out)[2][FB]) {
#pragma unroll
    for (int s = 0; s < NDS; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8 yop = rread(buf, is_y1, s, 2 * j + h, t);
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
          out[h][fb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(yop, xop[fb][s], out[h][fb], 0, 0, 0);
      }
  };

  // ---- the streamed loop: wait for tile t, start tile t+1, compute tile t ----
  // Steps come in pairs with fixed buffer roles (even tiles in stage 0, odd
  // in stage 1): with the stage chosen at run time the compiler cannot tell
  // a tile's LDS reads from the copy of the next tile in flight, and made
  // every wave wait for that copy before reading.
  auto step = [&](int t, const uint16_t* b1, const uint16_t* b2, const float4* srow,
                  uint16_t* n1, uint16_t* n2, float4* nrow) {
    // (made provably uniform: every wave-level decision below depends on them)
    const int sbase = __builtin_amdgcn_readfirstlane(tile_first(t));
    const int th = __builtin_amdgcn_readfirstlane(tile_head(t));
    wait_vmem();
    __syncthreads();
    if (t + 1 < n_st) {
      issue(t + 1, n1, n2);
      issue_rows(t + 1, nrow);
    }
    // (nothing of the tile's work is scheduled above the copies: hoisted
    // there, its LDS reads held registers across the copy code, and the D=64
    // dK/dV pass spilled)
    __builtin_amdgcn_sched_barrier(0);
    // does this wave see any (streamed, fixed) pair of the tile, and does the
    // tile need per-element masks?
    bool any = wave_active, need_mask;
    if constexpr (!KV) {
      const int wlast = min(fw0 + 16 * FB, nfixed) - 1;
      if (CAUSAL) any = any && sbase <= off + wlast;
      if (WINDOW) any = any && sbase + BN - 1 >= off + fw0 - a.window;
      need_mask = sbase + BN > kl || (CAUSAL && sbase + BN - 1 > off + fw0) ||
                  (WINDOW && sbase < off + wlast - a.window);
    } else {
      const int wlast = min(fw0 + 16 * FB, nfixed) - 1;
      if (CAUSAL) any = any && sbase + BN - 1 >= fw0 - off;
      if (WINDOW) any = any && sbase <= wlast - off + a.window;
      need_mask = sbase + BN > ql || (CAUSAL && sbase < wlast - off) ||
                  (WINDOW && sbase + BN - 1 > fw0 - off + a.window);
    }
    if (!any) return;
    // One 32-row chunk of the streamed tile at a time (its S and dP, P and dS,
    // and its part of the second products): a third of the registers of the
    // whole tile's scores at once.
#pragma unroll
    for (int j = 0; j < NKC; ++j) {
      // S from zero; for D=256, dP from -D of its query row, so that the
      // product leaves dP - D (one subtraction per score fewer: 2.5% faster
      // there, 1-2% slower for D=64 and 128, which keep the add)
      constexpr bool DINIT = D == 256;
      f32x4 sacc[2][FB], dpacc[2][FB];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
          sacc[h][fb] = f32x4{};
#pragma unroll
          for (int i = 0; i < 4; ++i)
            dpacc[h][fb][i] =
                !DINIT ? 0.0f
                : KV   ? reinterpret_cast<const float2*>(srow + 32 * j + 8 * grp + 4 * h + i)->y
                       : dfx[fb];
        }
      // (D=256: waves raise their priority while they issue MFMA blocks, as
      // in the forward; measured 2% faster for D=256, slower for D=64)
      if constexpr (D == 256) set_prio<2>();
      products(b1, true, x1op, j, t, sacc);
      products(b2, false, x2op, j, t, dpacc);
      if constexpr (D == 256) set_prio<0>();
      // P and dS of the chunk; the per-element visibility tests only on tiles
      // that need them (MK), as a branch of its own: folded into selects, they
      // ran on every tile and were about half of the D=64 passes' VALU work
      bf16x8 pb[FB], dsb[FB];
      auto p_ds = [&](auto mk) {
        constexpr bool MK = decltype(mk)::value;
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
          const int frow = fw0 + 16 * fb + c16;  // fixed row of this lane
          // the streamed rows [s_lo, s_hi] this fixed row sees (causal,
          // window); rows at or past s_end do not exist
          const int s_end = KV ? ql : kl;
          int s_lo = INT_MIN, s_hi = INT_MAX;
          if constexpr (KV) {
            if (CAUSAL) s_lo = frow - off;
            if (WINDOW) s_hi = frow - off + a.window;
          } else {
            if (WINDOW) s_lo = off + frow - a.window;
            if (CAUSAL) s_hi = off + frow;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int h = e >> 2, i = e & 3;
            const int srel = 32 * j + 8 * grp + 4 * h + i;  // streamed row in tile
            const int sr = sbase + srel;
            const float s = sacc[h][fb][i];
            float l2, dd;
            if constexpr (KV) {
              const float2 sv = *reinterpret_cast<const float2*>(srow + srel);
              l2 = sv.x;
              dd = sv.y;
            } else {
              l2 = l2f[fb];
              dd = dfx[fb];
            }
            const int qi = KV ? sr : frow, kj = KV ? frow : sr;
            bool vis = true;
            if constexpr (MK) vis = sr < s_end && sr >= s_lo && sr <= s_hi;
            float x;
            if constexpr (HAS_MASK) {
              const int mh = KV ? th : hf;
              const float m = mask_at<MASK>(a.mask, b * a.mask_sb + mh * a.mask_sh +
                                                        (int64_t)min(qi, ql - 1) * a.mask_sr +
                                                        min(kj, kl - 1));
              vis = vis && m != -INFINITY;
              x = __builtin_fmaf(s, a.c, kLog2e * m) - l2;
            } else {
              x = __builtin_fmaf(s, a.c, -l2);
            }
            const float p = (MK || HAS_MASK) ? (vis ? __builtin_amdgcn_exp2f(x) : 0.0f)
                                             : __builtin_amdgcn_exp2f(x);
            const float ds = p * (DINIT ? dpacc[h][fb][i] : dpacc[h][fb][i] + dd);  // dd = -D
            pb[fb][e] = (__bf16)p;
            dsb[fb][e] = (__bf16)ds;
            // (with a mask, one chunk's mask loads at a time: all of them in
            // flight at once would not fit the registers)
            if (HAS_MASK && e == 7) __builtin_amdgcn_sched_barrier(0);
          }
        }
      };
      if (need_mask) {
        // (an empty volatile asm: the compiler can neither speculate this
        // side nor merge the two into selects)
        asm volatile("");
        p_ds(BoolTag<true>{});
      } else {
        p_ds(BoolTag<false>{});
      }
      // second products of the chunk: dQ^T += Y1^T dS^T, or dK^T += Y1^T dS
      // and dV^T += Y2^T P
      if constexpr (D == 256) set_prio<2>();
#pragma unroll
      for (int da = 0; da < NDA; ++da) {
        const int d = dpart * NDA + da;
        const bf16x8 t1 = tread(b1, true, d, j, t);
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
          acc1[da][fb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t1, dsb[fb], acc1[da][fb], 0, 0, 0);
        if constexpr (KV) {
          const bf16x8 t2 = tread(b2, false, d, j, t);
#pragma unroll
          for (int fb = 0; fb < FB; ++fb)
            acc2[da][fb] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(t2, pb[fb], acc2[da][fb], 0, 0, 0);
        }
      }
      if constexpr (D == 256) set_prio<0>();
    }
  };
  // (the D=64 dK/dV pass with a mask or window has too few registers to keep
  // both stages' addresses: one step per iteration there)
  constexpr bool PAIRED = !(D == 64 && KV && (WINDOW || HAS_MASK));
  if (n_st > 0) {
    issue(0, y1s0, y2s0);
    issue_rows(0, srow0);
  }
  if constexpr (PAIRED) {
    for (int t = 0; t < n_st; t += 2) {
      step(t, y1s0, y2s0, srow0, y1s1, y2s1, srow1);
      if (t + 1 < n_st) step(t + 1, y1s1, y2s1, srow1, y1s0, y2s0, srow0);
    }
  } else {
    for (int t = 0; t < n_st; ++t) {
      const bool odd = t & 1;
      step(t, odd ? y1s1 : y1s0, odd ? y2s1 : y2s0, odd ? srow1 : srow0, odd ? y1s0 : y1s1,
           odd ? y2s0 : y2s1, odd ? srow0 : srow1);
    }
  }

  // ---- epilogue: scale and store (fixed row c16 of block fb, dims 16d + 4grp + i) ----
#pragma unroll
  for (int fb = 0; fb < FB; ++fb) {
    const int frow = fw0 + 16 * fb + c16;
    if (!(wave_active && frow < nfixed)) continue;
    uint16_t* d1 = (KV ? a.dk + kv_base : a.dq + qh_base) + (int64_t)frow * xr;
#pragma unroll
    for (int da = 0; da < NDA; ++da) {
      const int d = dpart * NDA + da;
      bf16x4 ov;
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(acc1[da][fb][i] * a.scale);
      *reinterpret_cast<bf16x4*>(d1 + 16 * d + 4 * grp) = ov;
    }
    if constexpr (KV) {
      uint16_t* d2 = a.dv + kv_base + (int64_t)frow * xr;
#pragma unroll
      for (int da = 0; da < NDA; ++da) {
        const int d = dpart * NDA + da;
        bf16x4 ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = (__bf16)acc2[da][fb][i];
        *reinterpret_cast<bf16x4*>(d2 + 16 * d + 4 * grp) = ov;
      }
    }
  }
  wait_vmem();  // no LDS copy may still be in flight when the workgroup ends
#endif
}

template <int D, int PASS, bool CAUSAL, bool WINDOW, int MASK>
hipError_t launch_bwd(const BwdArgs& a, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL((fa_bwd_kernel<D, PASS, CAUSAL, WINDOW, MASK>), dim3(grid),
                     dim3(64 * BwdCfg<D, PASS>::W), 0, stream, a);
  return hipGetLastError();
}

// The launches, in order: rows (L2, -D into dQ's rows), with sinks the
// per-head sum of the sink gradient's row terms, dK/dV (reads the rows'
// values), dQ (reads its rows' values, then overwrites the rows).
template <int D, bool CAUSAL, bool WINDOW, int MASK>
hipError_t dispatch_bwd(BwdArgs a, hipStream_t stream) {
  const int64_t qrows = (int64_t)a.B * a.H * a.ql;
  if (qrows > 0) {
    constexpr int RPB = 256 / (D / 8);
    const int64_t groups = (qrows + RPB - 1) / RPB;
    hipLaunchKernelGGL(fa_bwd_rows_kernel<D>, dim3((unsigned)std::min<int64_t>(groups, 1 << 16)),
                       dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.sinks) {
    // (every head, also with no rows: its gradient is then 0)
    hipLaunchKernelGGL(fa_bwd_sinks_kernel, dim3((unsigned)a.H), dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.kl > 0 && a.B > 0) {
    a.n_ftiles = (a.kl + fixed_rows<D, kBwdKV>() - 1) / fixed_rows<D, kBwdKV>();
    const hipError_t e = launch_bwd<D, kBwdKV, CAUSAL, WINDOW, MASK>(
        a, (unsigned)(a.n_ftiles * a.B * a.Hkv), stream);
    if (e != hipSuccess) return e;
  }
  if (a.ql > 0 && a.B > 0) {
    a.n_ftiles = (a.ql + fixed_rows<D, kBwdQ>() - 1) / fixed_rows<D, kBwdQ>();
    return launch_bwd<D, kBwdQ, CAUSAL, WINDOW, MASK>(a, (unsigned)(a.n_ftiles * a.B * a.H),
                                                      stream);
  }
  return hipSuccess;
}

template <int D, bool CAUSAL, bool WINDOW>
hipError_t dispatch_bwd_m(const BwdArgs& a, int mask, hipStream_t s) {
  switch (mask) {
    case kMaskF32: return dispatch_bwd<D, CAUSAL, WINDOW, kMaskF32>(a, s);
    case kMaskBF16: return dispatch_bwd<D, CAUSAL, WINDOW, kMaskBF16>(a, s);
    case kMaskBool: return dispatch_bwd<D, CAUSAL, WINDOW, kMaskBool>(a, s);
    default: return dispatch_bwd<D, CAUSAL, WINDOW, kNoMask>(a, s);
  }
}

template <int D>
hipError_t dispatch_bwd_d(const BwdArgs& a, bool causal, bool window, int mask, hipStream_t s) {
  if (window) return dispatch_bwd_m<D, true, true>(a, mask, s);
  return causal ? dispatch_bwd_m<D, true, false>(a, mask, s)
                : dispatch_bwd_m<D, false, false>(a, mask, s);
}

bool aligned_to(const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

// Shared host path of the backward entry points; window < 0: none (window >= 0
// requires causal). The mask is mask_dtype with batch and head strides in
// elements; its rows are contiguous (row stride kl).
int train_bwd(const void* q, const void* k, const void* v, const void* mask, int mask_dtype,
              int64_t mask_sb, int64_t mask_sh, const void* O, const float* L, const void* dO,
              int batch, int n_heads, int n_kv_heads, int ql, int kl, int head_dim, float scale,
              int causal, int window, void* dQ, void* dK, void* dV, void* stream,
              const int64_t* q_strides = nullptr, const int64_t* k_strides = nullptr,
              int64_t mask_sr = -1, const float* sinks = nullptr, float* dsinks = nullptr) {
  if (batch < 0 || ql < 0 || kl < 0 || n_heads < 1 || n_kv_heads < 1) return FA_ERR_BAD_SIZE;
  if (n_heads % n_kv_heads != 0) return FA_ERR_HEAD_GROUPING;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return FA_ERR_HEAD_DIM;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (window >= 0 && !causal) return FA_ERR_WINDOW;
  if (mask && ((mask_dtype != FA_MASK_F32 && mask_dtype != FA_MASK_BF16 &&
                mask_dtype != FA_MASK_BOOL) ||
               mask_sb < 0 || mask_sh < 0))
    return FA_ERR_MASK;
  // element strides (batch, head, row) of the Q-shaped and K-shaped tensors
  int64_t qs[3] = {(int64_t)n_heads * ql * head_dim, (int64_t)ql * head_dim, head_dim};
  int64_t ks[3] = {(int64_t)n_kv_heads * kl * head_dim, (int64_t)kl * head_dim, head_dim};
  for (int i = 0; i < 3; ++i) {
    if (q_strides) qs[i] = q_strides[i];
    if (k_strides) ks[i] = k_strides[i];
    if (qs[i] < 0 || ks[i] < 0) return FA_ERR_STRIDE;
    if (qs[i] % 8 != 0 || ks[i] % 8 != 0) return FA_ERR_ALIGNMENT;  // 16-byte rows
  }
  // a streamed tile's rows must lie within a 32-bit buffer offset
  if (qs[2] > (1 << 24) || ks[2] > (1 << 24)) return FA_ERR_TOO_LARGE;
  // dQ (Q's triple) and dK, dV (K's triple) are written: no two elements of
  // one may share an address (several workgroups would race on it)
  const int64_t qn[3] = {batch, n_heads, ql}, kn[3] = {batch, n_kv_heads, kl};
  if (view_overlaps(qs, qn, head_dim) || view_overlaps(ks, kn, head_dim)) return FA_ERR_STRIDE;
  const int64_t qrows = (int64_t)batch * n_heads * ql;
  const int64_t krows = (int64_t)batch * n_kv_heads * kl;
  if (sinks && !dsinks) return FA_ERR_NULL_POINTER;
  if ((sinks && !aligned_to(sinks, 4)) || (dsinks && sinks && !aligned_to(dsinks, 4)))
    return FA_ERR_ALIGNMENT;
  // (with sinks the heads' gradients are written even when there are no rows)
  if (qrows == 0 && krows == 0 && !sinks) return FA_OK;
  if (qrows > 0 && (!q || !O || !L || !dO || !dQ)) return FA_ERR_NULL_POINTER;
  if (krows > 0 && (!k || !v || !dK || !dV)) return FA_ERR_NULL_POINTER;
  if (qrows > 0 && krows > 0 && (!q || !k || !v)) return FA_ERR_NULL_POINTER;
  const void* a16[] = {q, k, v, O, dO, dQ, dK, dV};
  for (const void* p : a16)
    if (p && !aligned_to(p, 16)) return FA_ERR_ALIGNMENT;
  const uintptr_t mask_align = mask_dtype == FA_MASK_BF16 ? 2 : mask_dtype == FA_MASK_BOOL ? 1 : 4;
  if ((L && !aligned_to(L, 4)) || (mask && !aligned_to(mask, mask_align))) return FA_ERR_ALIGNMENT;
  const int64_t rq = head_dim == 64    ? fixed_rows<64, kBwdQ>()
                     : head_dim == 128 ? fixed_rows<128, kBwdQ>()
                                       : fixed_rows<256, kBwdQ>();
  const int64_t rk = head_dim == 64    ? fixed_rows<64, kBwdKV>()
                     : head_dim == 128 ? fixed_rows<128, kBwdKV>()
                                       : fixed_rows<256, kBwdKV>();
  if ((ql + rq - 1) / rq * batch * n_heads > 0x7fffffffLL ||
      (kl + rk - 1) / rk * batch * n_kv_heads > 0x7fffffffLL ||
      (int64_t)kl * head_dim * 2 > 0x7fffffffLL || (int64_t)ql * head_dim * 2 > 0x7fffffffLL)
    return FA_ERR_TOO_LARGE;

  BwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(O);
  a.dO = static_cast<const uint16_t*>(dO);
  a.L = L;
  a.mask = mask;
  a.mask_sb = mask_sb;
  a.mask_sh = mask_sh;
  a.mask_sr = mask_sr < 0 ? kl : (int)mask_sr;
  const int mask_kind = !mask                          ? kNoMask
                        : mask_dtype == FA_MASK_BF16 ? kMaskBF16
                        : mask_dtype == FA_MASK_BOOL ? kMaskBool
                                                     : kMaskF32;
  a.dq = static_cast<uint16_t*>(dQ);
  a.dk = static_cast<uint16_t*>(dK);
  a.dv = static_cast<uint16_t*>(dV);
  a.B = batch;
  a.H = n_heads;
  a.Hkv = n_kv_heads;
  a.ql = ql;
  a.kl = kl;
  a.group = n_heads / n_kv_heads;
  a.n_ftiles = 0;
  a.causal_off = kl > ql ? kl - ql : 0;
  // (a window past the largest q_abs hides nothing more; clamped there so that
  // q_abs - window stays in int range)
  a.window = window >= 0 ? (int)std::min<int64_t>(window, (int64_t)a.causal_off + ql) : 0;
  a.scale = scale;
  a.q_sb = qs[0], a.q_sh = qs[1], a.q_sr = (int)qs[2];
  a.k_sb = ks[0], a.k_sh = ks[1], a.k_sr = (int)ks[2];
  // a zero scale runs with the smallest normal exp2 factor (the scores it
  // produces round to 0, so P is the same uniform one); dQ and dK use the
  // true scale and come out 0
  const float c = scale * kLog2e;
  a.c = c == 0.0f ? FLT_MIN : c;
  a.sinks = sinks;
  a.dsinks = sinks ? dsinks : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool windowed = window >= 0;
  const hipError_t err =
      head_dim == 64    ? dispatch_bwd_d<64>(a, causal != 0, windowed, mask_kind, s)
      : head_dim == 128 ? dispatch_bwd_d<128>(a, causal != 0, windowed, mask_kind, s)
                        : dispatch_bwd_d<256>(a, causal != 0, windowed, mask_kind, s);
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" int fa_train_bwd(const void* q, const void* k, const void* v, const float* mask,
                            const void* O, const float* L, const void* dO, int batch, int n_heads,
                            int n_kv_heads, int ql, int kl, int head_dim, float scale, int causal,
                            void* dQ, void* dK, void* dV, void* stream) {
  const int64_t head = (int64_t)ql * kl;
  return train_bwd(q, k, v, mask, FA_MASK_F32, head * n_heads, head, O, L, dO, batch, n_heads,
                   n_kv_heads, ql, kl, head_dim, scale, causal, -1, dQ, dK, dV, stream);
}

extern "C" int fa_train_bwd_swa(const void* q, const void* k, const void* v, const float* mask,
                                const void* O, const float* L, const void* dO, int batch,
                                int n_heads, int n_kv_heads, int ql, int kl, int head_dim,
                                float scale, int window, void* dQ, void* dK, void* dV,
                                void* stream) {
  if (window < 0) return FA_ERR_WINDOW;
  const int64_t head = (int64_t)ql * kl;
  return train_bwd(q, k, v, mask, FA_MASK_F32, head * n_heads, head, O, L, dO, batch, n_heads,
                   n_kv_heads, ql, kl, head_dim, scale, 1, window, dQ, dK, dV, stream);
}

extern "C" int fa_train_bwd_ex(const void* q, const void* k, const void* v, const void* mask,
                               int mask_dtype, long long mask_stride_b, long long mask_stride_h,
                               const void* O, const float* L, const void* dO, int batch,
                               int n_heads, int n_kv_heads, int ql, int kl, int head_dim,
                               float scale, int causal, int window, void* dQ, void* dK, void* dV,
                               void* stream) {
  return train_bwd(q, k, v, mask, mask_dtype, mask_stride_b, mask_stride_h, O, L, dO, batch,
                   n_heads, n_kv_heads, ql, kl, head_dim, scale, causal, window < 0 ? -1 : window,
                   dQ, dK, dV, stream);
}

extern "C" int fa_train_bwd_strided(const void* q, const void* k, const void* v, const void* O,
                                    const float* L, const void* dO, const long long* q_strides,
                                    const long long* kv_strides, const void* mask,
                                    int mask_dtype, const long long* mask_strides, int batch,
                                    int n_heads,
                                    int n_kv_heads, int ql, int kl, int head_dim, float scale,
                                    int causal, int window, void* dQ, void* dK, void* dV,
                                    void* stream) {
  int64_t qs[3], ks[3];
  for (int i = 0; i < 3; ++i) {
    if (q_strides) qs[i] = q_strides[i];
    if (kv_strides) ks[i] = kv_strides[i];
  }
  const int64_t mhead = (int64_t)ql * kl;
  const int64_t ms[3] = {mask_strides ? mask_strides[0] : mhead * n_heads,
                         mask_strides ? mask_strides[1] : mhead,
                         mask_strides ? mask_strides[2] : kl};
  if (mask && (ms[2] < 0 || ms[2] > 0x7fffffffLL)) return FA_ERR_MASK;
  return train_bwd(q, k, v, mask, mask_dtype, ms[0], ms[1], O, L, dO, batch, n_heads, n_kv_heads,
                   ql, kl, head_dim, scale, causal, window, dQ, dK, dV, stream,
                   q_strides ? qs : nullptr, kv_strides ? ks : nullptr, ms[2]);
}

extern "C" int fa_train_bwd_sinks(const void* q, const void* k, const void* v, const void* O,
                                  const float* L, const void* dO, const long long* q_strides,
                                  const long long* kv_strides, const void* mask, int mask_dtype,
                                  const long long* mask_strides, int batch, int n_heads,
                                  int n_kv_heads, int ql, int kl, int head_dim, float scale,
                                  int causal, int window, const float* sinks, void* dQ, void* dK,
                                  void* dV, float* dsinks, void* stream) {
  int64_t qs[3], ks[3];
  for (int i = 0; i < 3; ++i) {
    if (q_strides) qs[i] = q_strides[i];
    if (kv_strides) ks[i] = kv_strides[i];
  }
  const int64_t mhead = (int64_t)ql * kl;
  const int64_t ms[3] = {mask_strides ? mask_strides[0] : mhead * n_heads,
                         mask_strides ? mask_strides[1] : mhead,
                         mask_strides ? mask_strides[2] : kl};
  if (mask && (ms[2] < 0 || ms[2] > 0x7fffffffLL)) return FA_ERR_MASK;
  return train_bwd(q, k, v, mask, mask_dtype, ms[0], ms[1], O, L, dO, batch, n_heads, n_kv_heads,
                   ql, kl, head_dim, scale, causal, window, dQ, dK, dV, stream,
                   q_strides ? qs : nullptr, kv_strides ? ks : nullptr, ms[2], sinks, dsinks);
}
