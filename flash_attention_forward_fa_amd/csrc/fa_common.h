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
__host__ __device__ __forceinline__ int key_of(int kb, int m) {
  return 32 * (kb >> 1) + 8 * (m >> 2) + 4 * (kb & 1) + (m & 3);
}

// LDS layouts (bf16, [key][d] in 16-byte chunks of 8 dims):
// Row-major widths (W = 64, 128, 256): chunk c of K row r sits at slot
// c ^ kswz<W>(r) of its row, chunk c of V row r at slot c ^ vswz<W>(r). The
// permutations were chosen by measuring LDS bank-conflict cycles
// (SQ_LDS_BANK_CONFLICT) for the exact access patterns of the kernels: the K
// rows one ds_read_b128 reaches (keys key_of(kb, 0..15)) and the V rows the
// 16-lane groups of one ds_read_b64_tr_b16 reach (four rows per group) all
// come out conflict-free with these, for 128-byte (W=64) and 512-byte (W=256)
// rows; 256-byte (W=128) rows use the W=256 permutations (any value below the
// row's 16 chunks is a valid permutation).
template <int W> __host__ __device__ __forceinline__ int kswz(int r) {
  return W == 64 ? ((r & 3) | ((r >> 1) & 4)) : ((r & 3) | ((r >> 1) & 12));
}
template <int W> __host__ __device__ __forceinline__ int vswz(int r) {
  return W == 64 ? 2 * (((r >> 1) & 1) | ((r >> 2) & 2)) : 2 * ((r & 3) | ((r >> 1) & 4));
}
// Other widths (W = 80, 96, 192; 64-key tiles only) are stored in panels: the
// dims [64i, 64i + 64) of all 64 rows form panel i, laid out exactly as a
// W=64 tile (so every read of a full panel meets the measured conflict-free
// pattern), followed by a tail panel of the last 16 or 32 dims. A tail of 2
// chunks per row keeps, in each aligned group of 16 slots, rows whose bits
// (0, 1, 3, 4) differ, with the chunk index flipping bit 3 of the slot; a tail
// of 4 chunks per row is row-major with the chunk index XORed by bits 1 and 3
// of the row. In a bank model of 64 four-byte banks (ds_read_b128 served 8
// lanes at a time, 64-bit reads 32 lanes at a time) both tails are read
// conflict-free by the K and V access patterns of the forward kernel.
template <int W> constexpr bool kPanels = !(W == 64 || W == 128 || W == 256);
__host__ __device__ __forceinline__ int tail2_slot(int r, int c) {
  const int h = ((r & 3) | (((r >> 3) & 3) << 2)) ^ (c << 3);
  const int q = ((r >> 2) & 1) | (((r >> 5) & 1) << 1) | (c << 2);
  return 16 * q + h;
}
__host__ __device__ __forceinline__ int tail4_swz(int r) { return ((r >> 1) & 1) | ((r >> 2) & 2); }
__host__ __device__ __forceinline__ int tail4_slot(int r, int c) { return 4 * r + (c ^ tail4_swz(r)); }
template <bool IS_K> __host__ __device__ __forceinline__ int swz64(int r) {
  return IS_K ? kswz<64>(r) : vswz<64>(r);
}

// Element offset, in a tile of width W, of the 16-byte piece of row r that
// holds dims [8c, 8c + 8).
template <int W, bool IS_K> __host__ __device__ __forceinline__ int lds_chunk(int r, int c) {
  if constexpr (!kPanels<W>) {
    return r * W + 8 * (c ^ (IS_K ? kswz<W>(r) : vswz<W>(r)));
  } else {
    constexpr int P = W / 64;
    if (c < 8 * P) return 4096 * (c >> 3) + 64 * r + 8 * ((c & 7) ^ swz64<IS_K>(r));
    return 4096 * P + 8 * (W % 64 == 16 ? tail2_slot(r, c - 8 * P) : tail4_slot(r, c - 8 * P));
  }
}
// The inverse: row r and chunk c stored in 16-byte slot p of the tile.
template <int W, bool IS_K> __host__ __device__ __forceinline__ void slot_chunk(int p, int& r, int& c) {
  if constexpr (!kPanels<W>) {
    r = p / (W / 8);
    c = (p % (W / 8)) ^ (IS_K ? kswz<W>(r) : vswz<W>(r));
  } else {
    constexpr int P = W / 64;
    if (p < 512 * P) {
      r = (p & 511) >> 3;
      c = 8 * (p >> 9) + ((p & 7) ^ swz64<IS_K>(r));
    } else if constexpr (W % 64 == 16) {
      const int t = p - 512 * P, q = t >> 4;
      const int cc = q >> 2, h = (t & 15) ^ (cc << 3);
      r = (h & 3) | ((q & 1) << 2) | (((h >> 2) & 3) << 3) | (((q >> 1) & 1) << 5);
      c = 8 * P + cc;
    } else {
      const int t = p - 512 * P;
      r = t >> 2;
      c = 8 * P + ((t & 3) ^ tail4_swz(r));
    }
  }
}

// Element offsets of the pieces the forward kernel's lanes read (with g the
// lane's 16-lane group and q4 = (lane & 15) & 3):
// the 16-byte K piece of row r for 32-dim step s (dims 32s + 8g .. + 7),
template <int W> __host__ __device__ __forceinline__ int k_step_piece(int r, int s, int g) {
  if constexpr (!kPanels<W>) {
    return r * W + 8 * ((4 * s + g) ^ kswz<W>(r));
  } else {
    constexpr int P = W / 64;
    return s < 2 * P ? 4096 * (s >> 1) + 64 * r + 8 * ((4 * (s & 1) + g) ^ kswz<64>(r))
                     : 4096 * P + 8 * tail4_slot(r, g);
  }
}
// the 8-byte K piece of row r in a 16-dim tail (dims 64P + 4g .. + 3),
template <int W> __host__ __device__ __forceinline__ int k_tail16_piece(int r, int g) {
  static_assert(W % 64 == 16, "a 16-dim tail");
  return 4096 * (W / 64) + 8 * tail2_slot(r, g >> 1) + 4 * (g & 1);
}
// and the 8-byte V piece of row r for 16-dim block d (dims 16d + 4q4 .. + 3).
template <int W> __host__ __device__ __forceinline__ int v_piece(int r, int d, int q4) {
  if constexpr (!kPanels<W>) {
    const int col = 16 * d + 4 * q4;
    return r * W + 8 * ((col >> 3) ^ vswz<W>(r)) + (col & 7);
  } else {
    constexpr int P = W / 64;
    if (d < 4 * P)
      return 4096 * (d >> 2) + 64 * r + 8 * ((2 * (d & 3) + (q4 >> 1)) ^ vswz<64>(r)) +
             4 * (q4 & 1);
    const int c = 2 * (d - 4 * P) + (q4 >> 1);
    return 4096 * P + 8 * (W % 64 == 16 ? tail2_slot(r, c) : tail4_slot(r, c)) + 4 * (q4 & 1);
  }
}

// Buffer resource word 3 for raw (untyped) buffer loads on gfx9-family parts.
constexpr int kRsrcWord3 = 0x00020000;

// Copy of one K or V tile (keys kbase .. kbase+BN-1, rows of W dims) from HBM
// straight into an LDS buffer with buffer_load_dwordx4 ... lds (no VGPR
// staging). Each thread moves 16-byte chunks; a wave writes 1 KiB of
// consecutive LDS slots per instruction, so the layout above is realised by
// choosing which global chunk each lane fetches. `off` holds this thread's
// byte offsets within a full tile (computed once by copy_offsets); the buffer
// descriptor is rebased on the tile so that the per-tile work is scalar. When
// the tile's slots are not a multiple of the workgroup, the last round is
// issued by the first waves only. A tile that runs past the last key repeats
// the last key's row (those keys are masked out).
template <int W, int BN, int NT>
struct CopyShape {
  static constexpr int CH = W / 8;                     // 16-byte chunks per row
  static constexpr int SLOTS = BN * CH;                // 16-byte slots per tile
  static constexpr int ROUNDS = (SLOTS + NT - 1) / NT; // chunks per thread (at most)
  static_assert(SLOTS % 64 == 0, "a tile must be whole wave instructions");
  static_assert(!kPanels<W> || BN == 64, "panel layouts hold 64-row tiles");
  // Rounds whose lanes' offsets repeat: with whole rounds of whole rows
  // (NT % CH == 0, no panels) and the row permutations of kswz/vswz, which
  // repeat every 32 rows, round u's lane reads the chunk of round u % PERIOD
  // (NT / CH) * (u - u % PERIOD) rows further on, a uniform offset; so only
  // PERIOD offsets per lane are kept in registers, the rest go as the scalar
  // offset. Used for 4-wave workgroups only (the head_dim-64 window kernels,
  // where it removed the spills); with 8 waves the registers were to spare
  // and the head_dim-128 forward ran 5% slower with it. (PERIOD = ROUNDS: one
  // register per round.)
  static constexpr int RPR = NT / CH;  // rows per round
  static constexpr int PERIOD =
      (NT != 256 || kPanels<W> || NT % CH != 0 || SLOTS % NT != 0) ? ROUNDS
      : RPR >= 32                                                   ? 1
                  : (32 / RPR < ROUNDS ? 32 / RPR : ROUNDS);
};

// (rs: the source's row stride in elements, W when its rows are contiguous)
template <int W, bool IS_K>
__device__ __forceinline__ int chunk_offset(int p, int row, int rs = W) {
  int r, c;
  slot_chunk<W, IS_K>(p, r, c);
  return (row * rs + 8 * c) * 2;
}

template <int W, int BN, int NT, bool IS_K>
__device__ __forceinline__ void copy_offsets(int tid, int (&off)[CopyShape<W, BN, NT>::ROUNDS],
                                             int rs = W) {
  constexpr int SLOTS = CopyShape<W, BN, NT>::SLOTS;
#pragma unroll
  for (int u = 0; u < CopyShape<W, BN, NT>::ROUNDS; ++u) {
    const int p = u * NT + tid;  // LDS slot (16-byte units)
    int r = 0, c = 0;
    if (SLOTS % NT == 0 || p < SLOTS) slot_chunk<W, IS_K>(p, r, c);
    off[u] = (r * rs + 8 * c) * 2;
  }
}

// (BRANCH: keep the partial-tile path a branch, below)
template <int W, int BN, int NT, bool IS_K, bool BRANCH = false>
__device__ __forceinline__ void issue_tile(const uint16_t* src, int kbase, int kl, uint16_t* lds,
                                           int tid, int wave_base,
                                           const int (&off)[CopyShape<W, BN, NT>::ROUNDS],
                                           int rs = W) {
  constexpr int ROUNDS = CopyShape<W, BN, NT>::ROUNDS;
  constexpr int SLOTS = CopyShape<W, BN, NT>::SLOTS;
  const int rows = kl - kbase;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(src + (int64_t)kbase * rs), 0, ((min(rows, BN) - 1) * rs + W) * 2, kRsrcWord3);
  constexpr int PERIOD = CopyShape<W, BN, NT>::PERIOD, RPR = CopyShape<W, BN, NT>::RPR;
  // (full tiles: round u's uniform part as the scalar offset, outside the
  // range check, which the lane's part, within round 0's rows, passes)
  if (rows >= BN) {
#pragma unroll
    for (int u = 0; u < ROUNDS; ++u)
      if ((u + 1) * NT <= SLOTS || u * NT + wave_base < SLOTS)  // (wave-uniform)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (lds_void*)(lds + (u * NT + wave_base) * 8), 16, off[u % PERIOD],
            (u - u % PERIOD) * RPR * rs * 2, 0, 0);
  } else {
    // (with BRANCH, an empty volatile asm keeps this rare path a branch:
    // speculated into the full-tile path as selects, its vector arithmetic
    // would run for every tile; the forward kernel takes it, the backward's
    // streaming loops have no registers to spare for it)
    if constexpr (BRANCH) asm volatile("");
#pragma unroll
    for (int u = 0; u < ROUNDS; ++u) {
      if ((u + 1) * NT <= SLOTS || u * NT + wave_base < SLOTS) {
        // (this thread's row moved back to the last valid one)
        int row, c;
        slot_chunk<W, IS_K>(u * NT + tid, row, c);
        // (the whole offset in the lane's register: the buffer's range check
        // sees only that part, and the clamped row may lie before round 0's)
        const int o = off[u % PERIOD] + ((u - u % PERIOD) * RPR - max(row - (rows - 1), 0)) * rs * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (lds_void*)(lds + (u * NT + wave_base) * 8), 16, o, 0, 0, 0);
      }
    }
  }
}

// A read of read-only int data at a wave-uniform index through the scalar
// cache (s_load): the constant address space tells the compiler the data is
// not written while the kernel runs. (A vector load here would have to wait,
// in order, behind every tile copy in flight.)
__device__ __forceinline__ int load_uniform(const int* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int*)(uintptr_t)p)[i];
}

// The same copy from a block-paged cache whose blocks may be shorter than a
// tile: block_size a positive multiple of 16 (row-major widths only). One
// wave instruction moves 64 chunks = 64 / (W / 8) consecutive tile rows (at
// most 8), which then lie in one block; its buffer descriptor is based at that
// block's row of the instruction's first row (a wave-uniform table read),
// clamped into the cache. Rows past the sequence's last key repeat that key's
// row, as above.
template <int W, int BN, int NT, bool IS_K>
__device__ __forceinline__ void issue_tile_blocks(const uint16_t* cache, const int* table_row,
                                                  int n_blocks, int n_kv_heads, int g,
                                                  int block_size, int kbase, int kl, uint16_t* lds,
                                                  int tid, int wave_base) {
  constexpr int CH = W / 8;
  constexpr int RPW = 64 / CH;  // rows per wave instruction
  constexpr int ROUNDS = CopyShape<W, BN, NT>::ROUNDS;
  static_assert(!kPanels<W> && ROUNDS * NT == BN * CH, "row-major whole-round tiles only");
  static_assert(RPW >= 1 && 16 % RPW == 0, "a wave instruction must stay in one 16-row block");
  const int rows = min(BN, kl - kbase);
#pragma unroll
  for (int u = 0; u < ROUNDS; ++u) {
    const int p = u * NT + tid;
    const int row0 = __builtin_amdgcn_readfirstlane((u * NT + wave_base) / CH);
    const int base_row = min(row0, rows - 1);
    const int pos = kbase + base_row;
    int blk = load_uniform(table_row, pos / block_size);
    blk = min(max(blk, 0), n_blocks - 1);
    const uint16_t* src =
        cache + (((int64_t)blk * n_kv_heads + g) * block_size + pos % block_size) * W;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, RPW * W * 2, kRsrcWord3);
    const int o = chunk_offset<W, IS_K>(p, min(p / CH, rows - 1)) - base_row * W * 2;
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
// vmcnt(N) (at most N vector memory loads of this wave still outstanding)
template <int N> __device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

}  // namespace
