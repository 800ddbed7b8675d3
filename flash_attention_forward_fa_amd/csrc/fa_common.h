// fa_common.h - device helpers shared by the forward and backward kernels
// (gfx950): vector types, reductions over the four 16-lane groups of a
// wave, the key permutation of the Q.K operand, the LDS chunk permutations,
// the direct-to-LDS tile copy, mask element reads and small scheduling
// helpers.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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
// group_max of two values at once: the first swap pairs the upper half of x
// with the lower half of y, so one max reduces x in lanes 0-31 and y in lanes
// 32-63; after the 16-lane step a last swap hands each half's result back to
// all lanes.
__device__ __forceinline__ void group_max2(float& x, float& y) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  const float h = __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const float f = swap16(h, true);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(f), __float_as_uint(f), false, false);
  x = __uint_as_float(b[0]);
  y = __uint_as_float(b[1]);
}
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
// (D=256) rows; 256-byte (D=128) rows use the D=256 permutations (any value
// below the row's 16 chunks is a valid permutation).
template <int D> __device__ __forceinline__ int kswz(int r) {
  return D == 64 ? ((r & 3) | ((r >> 1) & 4)) : ((r & 3) | ((r >> 1) & 12));
}
template <int D> __device__ __forceinline__ int vswz(int r) {
  return D == 64 ? 2 * (((r >> 1) & 1) | ((r >> 2) & 2)) : 2 * ((r & 3) | ((r >> 1) & 4));
}

// Buffer resource word 3 for raw (untyped) buffer loads on gfx9-family parts.
constexpr int kRsrcWord3 = 0x00020000;

// Copy of one K or V tile (keys kbase .. kbase+BN-1) from HBM straight into an
// LDS buffer with buffer_load_dwordx4 ... lds (no VGPR staging). Each thread
// moves 16-byte chunks; a wave writes 1 KiB of consecutive LDS per
// instruction, so a row's chunk permutation is realised by choosing which
// global chunk each lane fetches. `off` holds this thread's byte offsets
// within a full tile (computed once by copy_offsets); the buffer descriptor is
// rebased on the tile so that the per-tile work is scalar. A tile that runs
// past the last key repeats the last key's row (those keys are masked out).
template <int D, int BN, int NT>
struct CopyShape {
  static constexpr int CH = D / 8;             // 16-byte chunks per row
  static constexpr int ROUNDS = BN * CH / NT;  // chunks per thread
  static_assert(ROUNDS * NT == BN * CH, "tile not a multiple of the workgroup");
};

// (rs: the source's row stride in elements, D when its rows are contiguous)
template <int D, bool IS_K>
__device__ __forceinline__ int chunk_offset(int p, int row, int rs = D) {
  constexpr int CH = D / 8;
  const int r = p / CH;
  return (row * rs + 8 * ((p % CH) ^ (IS_K ? kswz<D>(r) : vswz<D>(r)))) * 2;
}

template <int D, int BN, int NT, bool IS_K>
__device__ __forceinline__ void copy_offsets(int tid, int (&off)[CopyShape<D, BN, NT>::ROUNDS],
                                             int rs = D) {
#pragma unroll
  for (int u = 0; u < CopyShape<D, BN, NT>::ROUNDS; ++u) {
    const int p = u * NT + tid;  // LDS slot (16-byte units)
    off[u] = chunk_offset<D, IS_K>(p, p / (D / 8), rs);
  }
}

template <int D, int BN, int NT, bool IS_K>
__device__ __forceinline__ void issue_tile(const uint16_t* src, int kbase, int kl, uint16_t* lds,
                                           int tid, int wave_base,
                                           const int (&off)[CopyShape<D, BN, NT>::ROUNDS],
                                           int rs = D) {
  constexpr int ROUNDS = CopyShape<D, BN, NT>::ROUNDS;
  const int rows = kl - kbase;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(src + (int64_t)kbase * rs), 0, ((min(rows, BN) - 1) * rs + D) * 2, kRsrcWord3);
  if (rows >= BN) {
#pragma unroll
    for (int u = 0; u < ROUNDS; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (lds_void*)(lds + (u * NT + wave_base) * 8), 16, off[u], 0, 0, 0);
  } else {
#pragma unroll
    for (int u = 0; u < ROUNDS; ++u) {
      // (this thread's row moved back to the last valid one)
      const int row = (u * NT + tid) / (D / 8);
      const int o = off[u] - max(row - (rows - 1), 0) * rs * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (lds_void*)(lds + (u * NT + wave_base) * 8), 16, o, 0, 0, 0);
    }
  }
}

// The same copy from a block-paged cache whose blocks may be shorter than a
// tile: block_size a positive multiple of 16. One wave instruction moves
// 64 chunks = 64 / (D / 8) consecutive tile rows (at most 8), which then lie
// in one block; its buffer descriptor is based at that block's row of the
// instruction's first row (a wave-uniform table read), clamped into the cache.
// Rows past the sequence's last key repeat that key's row, as above.
template <int D, int BN, int NT, bool IS_K>
__device__ __forceinline__ void issue_tile_blocks(const uint16_t* cache, const int* table_row,
                                                  int n_blocks, int n_kv_heads, int g,
                                                  int block_size, int kbase, int kl, uint16_t* lds,
                                                  int tid, int wave_base) {
  constexpr int CH = D / 8;
  constexpr int RPW = 64 / CH;  // rows per wave instruction
  constexpr int ROUNDS = CopyShape<D, BN, NT>::ROUNDS;
  static_assert(RPW >= 1 && 16 % RPW == 0, "a wave instruction must stay in one 16-row block");
  const int rows = min(BN, kl - kbase);
#pragma unroll
  for (int u = 0; u < ROUNDS; ++u) {
    const int p = u * NT + tid;
    const int row0 = __builtin_amdgcn_readfirstlane((u * NT + wave_base) / CH);
    const int base_row = min(row0, rows - 1);
    const int pos = kbase + base_row;
    int blk = __builtin_amdgcn_readfirstlane(table_row[pos / block_size]);
    blk = min(max(blk, 0), n_blocks - 1);
    const uint16_t* src =
        cache + (((int64_t)blk * n_kv_heads + g) * block_size + pos % block_size) * D;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, RPW * D * 2, kRsrcWord3);
    const int o = chunk_offset<D, IS_K>(p, min(p / CH, rows - 1)) - base_row * D * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + (u * NT + wave_base) * 8), 16,
                                             o, 0, 0, 0);
  }
}

// Mask element types (kNoMask: no mask): additive f32 or bf16, or boolean
// (one byte per key, nonzero = visible).
constexpr int kNoMask = 0, kMaskF32 = 1, kMaskBF16 = 2, kMaskBool = 3;

// Mask element idx as an additive f32 value (a bf16 mask widens exactly; a
// boolean mask is 0 for a visible key and -inf for a hidden one).
template <int MASK>
__device__ __forceinline__ float mask_at(const void* m, int64_t idx) {
  if constexpr (MASK == kMaskBF16)
    return __uint_as_float((uint32_t)static_cast<const uint16_t*>(m)[idx] << 16);
  else if constexpr (MASK == kMaskBool)
    return static_cast<const uint8_t*>(m)[idx] ? 0.0f : -INFINITY;
  else
    return static_cast<const float*>(m)[idx];
}

// Host check of an output view: n[0] x n[1] x n[2] rows (batch, head, row) of
// `row` contiguous elements at element strides st[0..2]. It maps two elements
// to one address unless, over the dimensions of size > 1 sorted by stride,
// every stride is at least the span of the dimensions below it (a sufficient
// condition for distinct addresses; interleaved layouts it cannot prove are
// rejected too).
inline bool view_overlaps(const int64_t st[3], const int64_t n[3], int64_t row) {
  if (row <= 0 || n[0] <= 0 || n[1] <= 0 || n[2] <= 0) return false;  // no elements
  int64_t ds[4], dn[4];
  int k = 0;
  if (row > 1) ds[k] = 1, dn[k++] = row;
  for (int i = 0; i < 3; ++i)
    if (n[i] > 1) ds[k] = st[i], dn[k++] = n[i];
  for (int i = 1; i < k; ++i)  // insertion sort by stride
    for (int j = i; j > 0 && ds[j] < ds[j - 1]; --j) {
      const int64_t t0 = ds[j], t1 = dn[j];
      ds[j] = ds[j - 1], dn[j] = dn[j - 1];
      ds[j - 1] = t0, dn[j - 1] = t1;
    }
  const int64_t kMax = INT64_MAX / 2;
  int64_t span = 1;
  for (int i = 0; i < k; ++i) {
    if (ds[i] < span) return true;
    // span of this and the lower dimensions, saturated (no address beyond it exists)
    span = ds[i] > (kMax - span) / (dn[i] - 1) ? kMax : ds[i] * (dn[i] - 1) + span;
  }
  return false;
}

// Wave priority for the next instructions, pinned in place.
template <int P> __device__ __forceinline__ void set_prio() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(P);
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void wait_vmem() {
  // vmcnt(0); expcnt and lgkmcnt left at their maxima
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

}  // namespace
