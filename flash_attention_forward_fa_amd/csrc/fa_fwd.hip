// fa_fwd.hip - flash-attention training forward (O and L) for AMD MI355X (gfx950).
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
// Work decomposition: one workgroup of 4 waves per (batch, head, 128 query
// rows); each wave owns 32 query rows (two blocks of 16). Per key tile, K and
// V are copied from HBM straight into LDS (global_load_lds_dwordx4, no VGPR
// staging) into one of two buffers while the previous tile is being computed.
// Every wave then computes, with v_mfma_f32_16x16x32_bf16,
//   S^T = K Q^T     (K rows read from LDS with ds_read_b128)
//   O^T += V^T P^T  (V^T read from the row-major V tile with ds_read_b64_tr_b16)
// so that in both products a lane holds one query row per 16-row block: row
// max, row sum and rescale are per-lane scalars after a reduction over the
// four 16-lane groups (v_permlane32_swap, v_permlane16_swap).
#include <hip/hip_runtime.h>

#include <float.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "fa.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Per head dim: QB 16-row query blocks per wave and BN keys per tile.
//   D=64:  2 blocks (32 rows per wave, 128 per workgroup), 64-key tiles.
//   D=256: 1 block (16 rows per wave, 64 per workgroup), 32-key tiles; the
//          O accumulator of 16 rows x 256 dims is 64 registers per lane, so
//          two workgroups share a compute unit.
template <int D> struct Cfg;
template <> struct Cfg<64> { static constexpr int QB = 2, BN = 64; };
template <> struct Cfg<256> { static constexpr int QB = 1, BN = 32; };
template <int D> constexpr int block_m() { return kWaves * 16 * Cfg<D>::QB; }

// A wave whose rows may see fewer keys than this starts with the compensated
// P.V product (P split into a bf16 high part and a bf16 remainder).
constexpr int kPreciseKeys = 128;
// After a plain pass, a row is recomputed compensated when |O| reaches this
// (one bf16 rounding step of O is then 2^-8 or more, and an error of the size
// of bf16(P)'s rounding can flip it) ...
constexpr float kRecheckO = 0.5f;
// ... or when its softmax is concentrated on so few keys (sum of the weights
// relative to the largest one below this) that the bf16 rounding of the
// row-sum terms does not average out.
constexpr float kRecheckL = 16.0f;
// The max used in exp2 is only raised when a tile's max exceeds it by more
// than this (base-2 units): P <= 2^kLazy and O is rarely rescaled.
constexpr float kLazy = 8.0f;

// Kernel modes. The plain kernel runs the bf16-P product and marks the rows
// that need the compensated product by writing kRowFlag into their L (their O
// is not written); the compensated kernel then recomputes exactly those rows
// (kFlagged), or every row when an additive mask is given (kAll).
constexpr int kPlain = 0, kAll = 1, kFlagged = 2;
constexpr uint32_t kRowFlag = 0x7FC0FA00u;  // a quiet NaN; never a valid L

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* mask;
  uint16_t* o;
  float* l;
  int B, H, Hkv, ql, kl;
  int group;       // H / Hkv
  int n_qtiles;    // ceil(ql / rows per workgroup)
  int causal_off;  // max(kl - ql, 0)
  float c;         // |scale| * log2(e), at least FLT_MIN
  uint32_t q_sign; // 0x80008000 flips the sign of both bf16 halves (scale < 0)
};

__device__ __forceinline__ float swap32(float x, bool take_max) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return take_max ? __builtin_fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float swap16(float x, bool take_max) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return take_max ? __builtin_fmaxf(a, b) : a + b;
}
// max / sum over the four 16-lane groups (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float group_max(float x) { return swap16(swap32(x, true), true); }
__device__ __forceinline__ float group_sum(float x) { return swap16(swap32(x, false), false); }

// Row of a 32-key chunk that lane row m of key block kb (16 keys) loads as the
// S^T A operand. With it, the four accumulators a lane of group g receives for
// blocks 2j and 2j+1 are keys 32j + 8g + (0..7): exactly the B-operand order
// of the P.V product, so P never moves between lanes.
__device__ __forceinline__ int key_of(int kb, int m) {
  return 32 * (kb >> 1) + 8 * (m >> 2) + 4 * (kb & 1) + (m & 3);
}

// LDS layouts (bf16, row-major [key][d], 16-byte chunks permuted per row):
// chunk c of K row r sits at slot c ^ kswz<D>(r), chunk c of V row r at slot
// c ^ vswz<D>(r). The permutations were chosen by measuring LDS bank-conflict
// cycles (SQ_LDS_BANK_CONFLICT) for the exact access patterns of this kernel:
// the K rows one ds_read_b128 reaches (keys key_of(kb, 0..15)) and the V rows
// the 16-lane groups of one ds_read_b64_tr_b16 reach (four rows per group)
// all come out conflict-free with these, for 128-byte (D=64) and 512-byte
// (D=256) rows.
template <int D> __device__ __forceinline__ int kswz(int r) {
  return D == 64 ? ((r & 3) | ((r >> 1) & 4)) : ((r & 3) | ((r >> 1) & 12));
}
template <int D> __device__ __forceinline__ int vswz(int r) {
  return D == 64 ? 2 * (((r >> 1) & 1) | ((r >> 2) & 2)) : 2 * ((r & 3) | ((r >> 1) & 4));
}

// Issue the copy of one K or V tile (rows kbase .. kbase+BN-1, clamped to the
// last valid row) from HBM into an LDS buffer. Each thread moves 16-byte
// chunks; a wave writes 1 KiB of consecutive LDS per instruction, so a row's
// chunk permutation is realised by choosing which global chunk each lane
// fetches.
template <int D, int BN, bool IS_K>
__device__ __forceinline__ void issue_tile(const uint16_t* src, int kbase, int kl, uint16_t* lds,
                                           int tid) {
  constexpr int CH = D / 8;  // chunks per row
  constexpr int ROUNDS = BN * CH / kThreads;
  const int wave_base = tid & ~63;
#pragma unroll
  for (int u = 0; u < ROUNDS; ++u) {
    const int p = u * kThreads + tid;  // LDS slot (16-byte units)
    const int r = p / CH;
    const int c = (p % CH) ^ (IS_K ? kswz<D>(r) : vswz<D>(r));
    const int key = min(kbase + r, kl - 1);
    const uint16_t* src_chunk = src + (int64_t)key * D + c * 8;
    __builtin_amdgcn_global_load_lds(src_chunk, (lds_void*)(lds + (u * kThreads + wave_base) * 8),
                                     16, 0, 0);
  }
}

__device__ __forceinline__ void wait_vmem() {
  // vmcnt(0); expcnt and lgkmcnt left at their maxima
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

template <int D, bool CAUSAL, bool HAS_MASK, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void fa_fwd_kernel(FwdArgs a) {
  static_assert(MODE != kPlain || !HAS_MASK, "the masked forward always runs compensated");
  constexpr bool PRECISE = MODE != kPlain;
  constexpr int BN = Cfg<D>::BN;
  constexpr int kQB = Cfg<D>::QB;
  constexpr int kRowsPerWave = 16 * kQB;
  constexpr int kBlockM = block_m<D>();
  constexpr int NKB = BN / 16;  // 16-key blocks per tile
  constexpr int NKC = BN / 32;  // 32-key chunks per tile (P.V contraction steps)
  constexpr int NDB = D / 16;   // 16-dim blocks of O
  constexpr int NDS = D / 32;   // 32-dim steps of Q.K
  constexpr int TILE = BN * D;  // elements per K or V tile
  __shared__ __attribute__((aligned(1024))) uint16_t k0s[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v0s[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k1s[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v1s[TILE];

  const int tid = threadIdx.x;
  // The wave index is made provably wave-uniform so that every condition
  // derived from it (tile skipping, compensated product, second pass) compiles
  // to a scalar branch: an MFMA left inside an EXEC-masked region still
  // accumulates (with whatever its operand registers hold) when EXEC is zero.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int c16 = lane & 15;  // query column within a 16-row block / A-operand row
  const int grp = lane >> 4;  // 16-lane group

  // ---- work item ----
  // Workgroups are handed to the 8 XCDs round-robin (bid mod 8). When B*H is a
  // multiple of 8, XCD x owns the heads [x*per, (x+1)*per) (so one KV group
  // stays within one XCD's L2) and walks its query tiles heaviest (most keys)
  // first across all its heads, so the cheap tiles fill the tail. (Running one
  // head at a time per XCD was measured slower.)
  const int BH = a.B * a.H;
  const int bid = blockIdx.x;
  int qt_rev, bh;
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, tl = bid >> 3, per = BH >> 3;
    qt_rev = tl / per;
    bh = xcd * per + tl % per;
  } else {
    qt_rev = bid / BH;
    bh = bid % BH;
  }
  const int qtile = a.n_qtiles - 1 - qt_rev;
  const int b = bh / a.H, h = bh % a.H;
  const int g = h / a.group;
  const int ql = a.ql, kl = a.kl, off = a.causal_off;
  const int q0 = qtile * kBlockM;
  const int qw0 = q0 + wave * kRowsPerWave;
  const int64_t kv_off = (int64_t)(b * a.Hkv + g) * kl * D;
  const uint16_t* kp = a.k + kv_off;
  const uint16_t* vp = a.v + kv_off;

  // ---- key range ----
  const int last_row = min(q0 + kBlockM, ql) - 1;
  const int kend = CAUSAL ? min(kl, off + last_row + 1) : kl;
  const int n_kt = (kend + BN - 1) / BN;
  const bool wave_active = qw0 < ql;
  const int wave_last = min(qw0 + kRowsPerWave, ql) - 1;
  const int wave_kend = CAUSAL ? min(kl, off + wave_last + 1) : kl;
  float* lrow_base = a.l + (int64_t)bh * ql;

  // ---- which rows this workgroup computes ----
  // Rows that may see fewer than kPreciseKeys keys (a property of their
  // position) always take the compensated product.
  auto short_rows = [&](int first_row) {
    return CAUSAL ? (min(kl, off + first_row + 1) < kPreciseKeys) : (kl < kPreciseKeys);
  };
  bool compute = wave_active;
  bool mine[kQB];  // kFlagged: this lane's row of block qb is to be recomputed
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) mine[qb] = false;
  if (MODE == kPlain) {
    if (short_rows(qw0)) {
      // hand these rows to the compensated kernel
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        const int qrow = qw0 + 16 * qb + c16;
        if (grp == 0 && qrow < ql) lrow_base[qrow] = __uint_as_float(kRowFlag);
      }
      compute = false;
    }
    // the last wave's rows start latest: if they are short, all are
    if (short_rows(q0 + (kWaves - 1) * kRowsPerWave)) return;
  } else if (MODE == kFlagged) {
    bool any = false;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const int qrow = qw0 + 16 * qb + c16;
      if (qrow < ql) mine[qb] = __float_as_uint(lrow_base[qrow]) == kRowFlag;
      any |= mine[qb];
    }
    compute = __any(any);
    if (!__syncthreads_or(compute)) return;
  }
  if (n_kt > 0) {
    issue_tile<D, BN, true>(kp, 0, kl, k0s, tid);
    issue_tile<D, BN, false>(vp, 0, kl, v0s, tid);
  }

  // ---- Q^T as the B operand: block qb, step s: row qw0+16qb+c16, dims 32s+8grp.. ----
  bf16x8 qop[kQB][NDS];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int qrow = min(qw0 + 16 * qb + c16, ql - 1);
    const uint16_t* qp = a.q + ((int64_t)bh * ql + qrow) * D + 8 * grp;
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
      u32x4 raw = *reinterpret_cast<const u32x4*>(qp + 32 * s);
      raw ^= a.q_sign;
      qop[qb][s] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  float m_use[kQB], m_top[kQB], l_run[kQB];
  f32x4 oacc[NDB][kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    m_use[qb] = -FLT_MAX / 2.0f;  // max used in exp2 (base 2)
    m_top[qb] = -FLT_MAX / 2.0f;  // true running max (base 2)
    l_run[qb] = 0.0f;             // this lane's partial row sum
#pragma unroll
    for (int d = 0; d < NDB; ++d) oacc[d][qb] = f32x4{};
  }

  // One key tile: wait for its copy, start the next one, compute.
  auto step = [&](int kt, const uint16_t* ks, const uint16_t* vs, uint16_t* nks, uint16_t* nvs) {
    const int kbase = kt * BN;
    wait_vmem();
    __syncthreads();
    if (kt + 1 < n_kt) {
      issue_tile<D, BN, true>(kp, kbase + BN, kl, nks, tid);
      issue_tile<D, BN, false>(vp, kbase + BN, kl, nvs, tid);
    }
    if (!compute || kbase >= wave_kend) return;

    // ---- S^T = K Q^T (raw scores, f32) ----
    f32x4 sacc[NKB][kQB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) sacc[kb][qb] = f32x4{};
#pragma unroll
    for (int s = 0; s < NDS; ++s)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int r = key_of(kb, c16);
        const int chunk = 4 * s + grp;
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(ks + r * D + 8 * (chunk ^ kswz<D>(r)));
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          sacc[kb][qb] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[qb][s], sacc[kb][qb], 0, 0, 0);
        // D=256: keep the scheduler from hoisting all K reads (register pressure)
        if (D == 256 && kb == NKB - 1 && (s & 1) == 1) __builtin_amdgcn_sched_barrier(0);
      }

    // ---- masks: tail keys, causal, additive ----
    if (HAS_MASK) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        const int qrow = qw0 + 16 * qb + c16;
        const float* mrow = a.mask + ((int64_t)bh * ql + min(qrow, ql - 1)) * kl;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kbase + 32 * (kb >> 1) + 8 * grp + 4 * (kb & 1) + i;
            const bool vis = key < kl && (!CAUSAL || key <= off + qrow);
            sacc[kb][qb][i] =
                vis ? __builtin_fmaf(sacc[kb][qb][i], a.c, kLog2e * mrow[key]) : -INFINITY;
          }
      }
    } else if ((kbase + BN > kl) || (CAUSAL && kbase + BN - 1 > off + qw0)) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        const int qabs = off + qw0 + 16 * qb + c16;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kbase + 32 * (kb >> 1) + 8 * grp + 4 * (kb & 1) + i;
            if (key >= kl || (CAUSAL && key > qabs)) sacc[kb][qb][i] = -INFINITY;
          }
      }
    }

    // ---- online softmax (base 2), lazy rescale ----
    // (the decision to raise is taken per row, so a row's result never
    // depends on its neighbours' scores)
    float m_new[kQB];
    bool raise = false;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = __builtin_fmaxf(mx, sacc[kb][qb][i]);
      mx = group_max(mx);
      const float tmax = HAS_MASK ? mx : mx * a.c;  // c > 0: max(c*r) == c*max(r)
      m_top[qb] = __builtin_fmaxf(m_top[qb], tmax);
      const bool r = tmax > m_use[qb] + kLazy;
      m_new[qb] = r ? tmax : m_use[qb];
      raise |= r;
    }
    if (__any(raise)) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        const float alpha = __builtin_amdgcn_exp2f(m_use[qb] - m_new[qb]);
        m_use[qb] = m_new[qb];
        l_run[qb] *= alpha;
#pragma unroll
        for (int d = 0; d < NDB; ++d) oacc[d][qb] *= alpha;
      }
    }

    // ---- P = exp2(s - m) in bf16 (+ remainder when compensated), row sums ----
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    bf16x8 phi[NKC][kQB], plo[NKC][kQB];
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
          p[e] = __builtin_amdgcn_exp2f(HAS_MASK ? sv + mneg : __builtin_fmaf(sv, a.c, mneg));
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

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int j = 0; j < NKC; ++j) {
        // V^T operand: dims 16d + c16, keys 32j + 8grp + (0..7), from two
        // transposing reads of four keys each
        s16x4 half[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int r = 32 * j + 8 * grp + 4 * t + (c16 >> 2);
          const int col = 16 * d + 4 * (c16 & 3);
          const uint16_t* addr = vs + r * D + 8 * ((col >> 3) ^ vswz<D>(r)) + (col & 7);
          half[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)addr);
        }
        const bf16x8 vop = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
          oacc[d][qb] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, phi[j][qb], oacc[d][qb], 0, 0, 0);
          if (PRECISE)
            oacc[d][qb] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, plo[j][qb], oacc[d][qb], 0, 0, 0);
        }
        // D=256: the same for the V reads
        if (D == 256 && j == NKC - 1 && (d & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
  };

  for (int kt = 0; kt < n_kt; ++kt) {
    const bool odd = kt & 1;
    step(kt, odd ? k1s : k0s, odd ? v1s : v0s, odd ? k0s : k1s, odd ? v0s : v1s);
  }

  // ---- epilogue: O = O_acc / l (+0 for an empty row), L = (m + log2 l) ln 2 ----
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int qrow = qw0 + 16 * qb + c16;
    const bool row_ok = compute && qrow < ql;
    const float l_tot = group_sum(l_run[qb]);
    bool write = row_ok;
    if (MODE == kPlain) {
      // rows whose plain result is not accurate enough go to the compensated kernel
      float omax = 0.0f;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) omax = __builtin_fmaxf(omax, __builtin_fabsf(oacc[d][qb][i]));
      omax = group_max(omax);
      const float l_rel = l_tot * __builtin_amdgcn_exp2f(m_use[qb] - m_top[qb]);
      const bool need = row_ok && l_tot > 0.0f && (omax >= kRecheckO * l_tot || l_rel < kRecheckL);
      if (need && grp == 0) lrow_base[qrow] = __uint_as_float(kRowFlag);
      write = row_ok && !need;
    } else if (MODE == kFlagged) {
      write = row_ok && mine[qb];
    }
    if (write) {
      const bool empty = !(l_tot > 0.0f);
      const float inv = empty ? 0.0f : __builtin_amdgcn_rcpf(l_tot);
      uint16_t* orow = a.o + ((int64_t)bh * ql + qrow) * D + 4 * grp;
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        bf16x4 ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = empty ? (__bf16)0.0f : (__bf16)(oacc[d][qb][i] * inv);
        *reinterpret_cast<bf16x4*>(orow + 16 * d) = ov;
      }
      if (grp == 0)
        lrow_base[qrow] = empty ? -INFINITY : (m_use[qb] + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
  }
  wait_vmem();  // no LDS copy may still be in flight when the workgroup ends
}

template <int D, bool CAUSAL, bool HAS_MASK, int MODE>
hipError_t launch(const FwdArgs& a, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, HAS_MASK, MODE>), dim3(grid), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

// Masked: one compensated launch. Unmasked: the plain launch, then the
// compensated launch for the rows it flagged (same stream, so in order).
template <int D, bool CAUSAL>
hipError_t dispatch_c(const FwdArgs& a, bool has_mask, unsigned grid, hipStream_t stream) {
  if (has_mask) return launch<D, CAUSAL, true, kAll>(a, grid, stream);
  hipError_t e = launch<D, CAUSAL, false, kPlain>(a, grid, stream);
  if (e != hipSuccess) return e;
  return launch<D, CAUSAL, false, kFlagged>(a, grid, stream);
}

template <int D>
hipError_t dispatch_d(const FwdArgs& a, bool causal, bool has_mask, unsigned grid,
                      hipStream_t stream) {
  return causal ? dispatch_c<D, true>(a, has_mask, grid, stream)
                : dispatch_c<D, false>(a, has_mask, grid, stream);
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

}  // namespace

extern "C" int fa_train_fwd(const void* q, const void* k, const void* v, const float* mask,
                            int batch, int n_heads, int n_kv_heads, int ql, int kl, int head_dim,
                            float scale, int causal, void* O, float* L, void* stream) {
  if (batch < 0 || ql < 0 || kl < 0 || n_heads < 1 || n_kv_heads < 1) return FA_ERR_BAD_SIZE;
  if (n_heads % n_kv_heads != 0) return FA_ERR_HEAD_GROUPING;
  if (head_dim != 64 && head_dim != 256) return FA_ERR_HEAD_DIM;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  const int64_t rows = (int64_t)batch * n_heads * ql;
  if (rows == 0) return FA_OK;
  const bool kv_used = kl > 0;
  if (!q || !O || !L || (kv_used && (!k || !v))) return FA_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(O, 16) || !aligned(L, 4) ||
      (kv_used && (!aligned(k, 16) || !aligned(v, 16))) || (mask && !aligned(mask, 4)))
    return FA_ERR_ALIGNMENT;
  const int bm = head_dim == 64 ? block_m<64>() : block_m<256>();
  const int64_t n_qtiles = ((int64_t)ql + bm - 1) / bm;
  const int64_t grid = n_qtiles * batch * n_heads;
  if (grid > 0x7fffffffLL || (int64_t)batch * n_heads > 0x7fffffffLL) return FA_ERR_TOO_LARGE;

  FwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.mask = mask;
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
  // Masked keys are carried as raw score -inf and scaled inside the kernel, which
  // needs c > 0; a zero scale is run as the smallest normal one (the scores it
  // produces round to 0 in f32, so the weights are the same uniform ones).
  a.c = fmaxf(fabsf(scale) * kLog2e, FLT_MIN);
  a.q_sign = signbit(scale) ? 0x80008000u : 0u;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = head_dim == 64 ? dispatch_d<64>(a, causal != 0, mask != nullptr, (unsigned)grid, s)
                                  : dispatch_d<256>(a, causal != 0, mask != nullptr, (unsigned)grid, s);
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case FA_ERR_BAD_SIZE: return "invalid size (batch, ql, kl < 0 or head counts < 1)";
    case FA_ERR_HEAD_GROUPING: return "n_heads is not a multiple of n_kv_heads";
    case FA_ERR_HEAD_DIM: return "head_dim must be 64 or 256";
    case FA_ERR_SCALE: return "scale must be finite";
    case FA_ERR_ALIGNMENT: return "misaligned tensor (q, k, v, O need 16 bytes; mask, L 4 bytes)";
    case FA_ERR_TOO_LARGE: return "problem too large for the kernel's grid or index range";
    case FA_ERR_LAUNCH: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}
