// fa_fwd.hip - flash-attention training forward (O and L) for AMD MI355X (gfx950).
//
// What is computed is fixed by the CPU oracle of the method's page
// ("mlx-native 0.9.0", tests/test_flash_attn_train.rs, doc comment and section
// "CPU oracle - forward O + logsumexp L"): per query row, base-2 scores
// s = scale*log2(e)*<q,k> (+ log2(e)*mask), bottom-right causal masking with the
// offset max(kl - ql, 0), a row max seeded with the finite sentinel -FLT_MAX/2,
// p = exp2(s - m), L = m*ln2 + ln(sum p), O = sum(p v) / sum p, and O = 0,
// L = -inf for a row with no visible key. The kernel reaches the same values
// tile by tile with an online (streaming) softmax over key tiles.
//
// Work decomposition: one workgroup of 4 waves per (batch, head, 128 query
// rows); each wave owns 32 query rows. Per key tile of 64 keys, K is staged in
// LDS as [key][d] and V as its transpose [d][key]; every wave then computes
//   S^T = K Q^T    (v_mfma_f32_32x32x16_bf16: 32 keys x 32 queries per block)
//   O^T += V^T P^T (same instruction: 32 head-dims x 32 queries per block)
// so that in both products lane l holds query row (l mod 32): the row max,
// the row sum and the O rescale are per-lane scalars, and the only cross-lane
// step is one v_permlane32_swap between the two half-waves.
#include <hip/hip_runtime.h>

#include <float.h>
#include <math.h>
#include <stdint.h>

#include "fa.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBlockM = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kBlockN = 64;                     // keys per tile
constexpr int kPad = 8;                         // bf16 padding per LDS row
// A wave whose rows may see fewer keys than this uses the compensated P.V
// product (P split into a bf16 high part and a bf16 remainder).
constexpr int kPreciseKeys = 128;
// ... and so does a wave in which some output row reaches this magnitude
// after the plain pass: from |O| = 0.5 on, one bf16 rounding step of O is
// 2^-8 or more, and a pre-rounding error of bf16(P) size flips it.
constexpr float kRecheckO = 0.5f;

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
  int n_qtiles;    // ceil(ql / kBlockM)
  int causal_off;  // max(kl - ql, 0)
  float c;         // |scale| * log2(e), at least FLT_MIN
  uint32_t q_sign; // 0x80008000 flips the sign of both bf16 halves (scale < 0)
};

__device__ __forceinline__ float wave_half_swap_max(float x) {
  // lanes l and l^32 exchange values; each keeps the larger
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row (key) of the K tile that lane row m of a 32-key block loads: bits 2 and
// 3 swapped. With this order the 16 accumulators a lane receives from the
// 32x32 product hold, per 8-register group, 8 consecutive keys
// (key = 16*(i/8) + 8*(lane/32) + i%8), which is exactly the B-operand order
// the P.V product needs.
__device__ __forceinline__ int key_perm(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <int D, bool CAUSAL, bool HAS_MASK>
__global__ __launch_bounds__(kThreads) void fa_fwd_kernel(FwdArgs a) {
  constexpr int DCH = D / 8;           // 16-byte chunks per K/V row
  constexpr int KS = D + kPad;         // LDS row stride of K (elements)
  constexpr int VS = kBlockN + kPad;   // LDS row stride of V^T (elements)
  constexpr int NKB = kBlockN / 32;    // 32-key blocks per tile
  constexpr int NDB = D / 32;          // 32-dim blocks of O
  constexpr int NQS = D / 16;          // 16-dim steps of Q.K
  __shared__ __attribute__((aligned(16))) uint16_t ks[kBlockN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * VS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;   // query row within the wave
  const int hh = lane >> 5;  // half-wave

  // ---- work item: heaviest causal tiles first; heads grouped per XCD ----
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
  const int qrow = qw0 + n;
  const bool row_ok = qrow < ql;
  const int qrow_c = row_ok ? qrow : ql - 1;

  const uint16_t* qp = a.q + ((int64_t)bh * ql + qrow_c) * D;
  const int64_t kv_off = (int64_t)(b * a.Hkv + g) * kl * D;
  const uint16_t* kp = a.k + kv_off;
  const uint16_t* vp = a.v + kv_off;

  // ---- Q^T as the B operand: lane holds row qrow, dims 16s + 8hh .. +7 ----
  bf16x8 qop[NQS];
#pragma unroll
  for (int s = 0; s < NQS; ++s) {
    u32x4 raw = *reinterpret_cast<const u32x4*>(qp + 16 * s + 8 * hh);
    raw ^= a.q_sign;
    qop[s] = __builtin_bit_cast(bf16x8, raw);
  }

  // ---- key range ----
  const int last_row = (q0 + kBlockM < ql ? q0 + kBlockM : ql) - 1;
  int kend = kl;
  if (CAUSAL) kend = min(kl, off + last_row + 1);
  const int n_kt = (kend + kBlockN - 1) / kBlockN;
  const bool wave_active = qw0 < ql;
  const int wave_last = min(qw0 + kRowsPerWave, ql) - 1;
  const int wave_kend = CAUSAL ? min(kl, off + wave_last + 1) : kl;
  // P.V precision: the plain product rounds P to bf16; the compensated one adds
  // the bf16 remainder P - bf16(P) in a second MFMA. Waves whose rows may see
  // few keys (by position only) and the masked variant start compensated. In
  // any other wave, a row whose plain result reaches |O| >= kRecheckO is
  // recomputed by a compensated second pass over the keys; every other row
  // keeps its first-pass result, so a row's output never depends on the data
  // of its neighbours.
  bool precise =
      HAS_MASK || (CAUSAL ? (min(kl, off + qw0 + 1) < kPreciseKeys) : (kl < kPreciseKeys));
  bool compute = wave_active;
  bool redo_row = false;  // this lane's row is rewritten by the second pass

  float m_run = -FLT_MAX / 2.0f;  // running max, base-2 units
  float l_run = 0.0f;             // this lane's partial row sum
  f32x16 oacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) oacc[d] = f32x16{};

  for (int pass = 0; pass < 2; ++pass) {
  for (int kt = 0; kt < n_kt; ++kt) {
    const int kbase = kt * kBlockN;
    __syncthreads();
    // ---- stage K tile [key][d] ----
#pragma unroll
    for (int c = tid; c < kBlockN * DCH; c += kThreads) {
      const int row = c / DCH, ch = c % DCH;
      const int key = kbase + row;
      u32x4 val = u32x4{};
      if (key < kl) val = *reinterpret_cast<const u32x4*>(kp + (int64_t)key * D + ch * 8);
      *reinterpret_cast<u32x4*>(ks + row * KS + ch * 8) = val;
    }
    // ---- stage V tile transposed [d][key], two keys per 32-bit LDS word ----
#pragma unroll
    for (int u = tid; u < (kBlockN / 2) * DCH; u += kThreads) {
      const int pr = u / DCH, ch = u % DCH;
      const int key0 = kbase + 2 * pr;
      u32x4 v0 = u32x4{}, v1 = u32x4{};
      if (key0 < kl) v0 = *reinterpret_cast<const u32x4*>(vp + (int64_t)key0 * D + ch * 8);
      if (key0 + 1 < kl) v1 = *reinterpret_cast<const u32x4*>(vp + (int64_t)(key0 + 1) * D + ch * 8);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t w0 = v0[j >> 1], w1 = v1[j >> 1];
        const uint32_t word = (j & 1) ? ((w0 >> 16) | (w1 & 0xFFFF0000u))
                                      : ((w0 & 0xFFFFu) | (w1 << 16));
        *reinterpret_cast<uint32_t*>(vt + (ch * 8 + j) * VS + 2 * pr) = word;
      }
    }
    __syncthreads();
    if (!compute || kbase >= wave_kend) continue;

    // ---- S^T = K Q^T (raw scores, f32) ----
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = f32x16{};
      const uint16_t* krow = ks + (32 * kb + key_perm(n)) * KS + 8 * hh;
#pragma unroll
      for (int s = 0; s < NQS; ++s) {
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(krow + 16 * s);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[s], sacc[kb], 0, 0, 0);
      }
    }

    // ---- masks: tail keys, causal, additive ----
    const int qabs = off + qrow;
    if (HAS_MASK) {
      const float* mrow = a.mask + ((int64_t)bh * ql + qrow_c) * kl;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kbase + 32 * kb + 16 * (i >> 3) + 8 * hh + (i & 7);
          const bool vis = key < kl && (!CAUSAL || key <= qabs);
          sacc[kb][i] = vis ? __builtin_fmaf(sacc[kb][i], a.c, kLog2e * mrow[key]) : -INFINITY;
        }
    } else {
      const bool edge = (kbase + kBlockN > kl) || (CAUSAL && kbase + kBlockN - 1 > off + qw0);
      if (edge) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kbase + 32 * kb + 16 * (i >> 3) + 8 * hh + (i & 7);
            const bool vis = key < kl && (!CAUSAL || key <= qabs);
            if (!vis) sacc[kb][i] = -INFINITY;
          }
      }
    }

    // ---- online softmax (base 2) ----
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, sacc[kb][i]);
    mx = wave_half_swap_max(mx);
    // scale is applied in f32 here (c > 0, so max(c*r) == c*max(r))
    const float m_new = __builtin_fmaxf(m_run, HAS_MASK ? mx : mx * a.c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float x = HAS_MASK ? sacc[kb][i] - m_new : __builtin_fmaf(sacc[kb][i], a.c, -m_new);
        const float p = __builtin_amdgcn_exp2f(x);
        sacc[kb][i] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8 phi;
#pragma unroll
        for (int e = 0; e < 8; ++e) phi[e] = (__bf16)sacc[kb][8 * half + e];
        const uint16_t* vcol = vt + n * VS + 32 * kb + 16 * half + 8 * hh;
        if (precise) {
          bf16x8 plo;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            plo[e] = (__bf16)(sacc[kb][8 * half + e] - (float)phi[e]);
#pragma unroll
          for (int d = 0; d < NDB; ++d) {
            const bf16x8 vop = *reinterpret_cast<const bf16x8*>(vcol + 32 * d * VS);
            oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, phi, oacc[d], 0, 0, 0);
            oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, plo, oacc[d], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int d = 0; d < NDB; ++d) {
            const bf16x8 vop = *reinterpret_cast<const bf16x8*>(vcol + 32 * d * VS);
            oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, phi, oacc[d], 0, 0, 0);
          }
        }
      }
  }
    // ---- finish the pass: rows that are final write O and L ----
    const float l_tot = wave_half_swap_sum(l_run);
    bool need = false;
    if (pass == 0 && compute && !precise) {
      float omax = 0.0f;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) omax = __builtin_fmaxf(omax, __builtin_fabsf(oacc[d][i]));
      omax = wave_half_swap_max(omax);  // max |O_acc| of this lane's row
      need = row_ok && l_tot > 0.0f && omax >= kRecheckO * l_tot;
    }
    if (row_ok && (pass == 0 ? !need : redo_row)) {
      // O = O_acc / l (+0 for an empty row), L = (m + log2 l) ln 2
      const bool empty = !(l_tot > 0.0f);
      const float inv = empty ? 0.0f : __builtin_amdgcn_rcpf(l_tot);
      uint16_t* orow = a.o + ((int64_t)bh * ql + qrow) * D;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          bf16x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            ov[e] = empty ? (__bf16)0.0f : (__bf16)(oacc[d][4 * g4 + e] * inv);
          *reinterpret_cast<bf16x4*>(orow + 32 * d + 8 * g4 + 4 * hh) = ov;
        }
      if (hh == 0)
        a.l[(int64_t)bh * ql + qrow] =
            empty ? -INFINITY : (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
    if (pass == 1) break;
    // ---- compensated second pass for the waves that have such rows ----
    redo_row = need;
    const bool wave_redo = __any(need);
    if (!__syncthreads_or(wave_redo)) break;
    compute = wave_redo;
    if (wave_redo) {
      precise = true;
      m_run = -FLT_MAX / 2.0f;
      l_run = 0.0f;
#pragma unroll
      for (int d = 0; d < NDB; ++d) oacc[d] = f32x16{};
    }
  }
}

template <int D, bool CAUSAL, bool HAS_MASK>
hipError_t launch(const FwdArgs& a, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, HAS_MASK>), dim3(grid), dim3(kThreads), 0, stream,
                     a);
  return hipGetLastError();
}

template <int D>
hipError_t dispatch_d(const FwdArgs& a, bool causal, bool has_mask, unsigned grid,
                      hipStream_t stream) {
  if (causal)
    return has_mask ? launch<D, true, true>(a, grid, stream) : launch<D, true, false>(a, grid, stream);
  return has_mask ? launch<D, false, true>(a, grid, stream) : launch<D, false, false>(a, grid, stream);
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
  const int64_t n_qtiles = ((int64_t)ql + kBlockM - 1) / kBlockM;
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
