// Host-side checks of the LDS tile layouts in fa_common.h (no GPU needed):
// for every row width, each layout is a bijection between (row, 16-byte chunk)
// and the tile's slots, slot_chunk is its inverse, and the per-lane piece
// addresses the kernels compute (k_step_piece, k_tail16_piece, v_piece) agree
// with lds_chunk. It also reports, for a bank model of 64 four-byte banks
// (ds_read_b128 served 8 lanes at a time, 64-bit reads 32 lanes at a time),
// the largest number of accesses of one pass that meet in one bank ("model"
// lines): the panel widths were designed for 1. Prints "ok" or the first
// failure and exits nonzero.
#include <stdio.h>
#include <string.h>

#include "fa_common.h"

template <int W, bool IS_K> static bool check_layout() {
  constexpr int CH = W / 8, SLOTS = 64 * CH;
  static bool seen[SLOTS];
  memset(seen, 0, sizeof(seen));
  for (int r = 0; r < 64; ++r)
    for (int c = 0; c < CH; ++c) {
      const int e = lds_chunk<W, IS_K>(r, c);
      if (e % 8 != 0 || e < 0 || e / 8 >= SLOTS || seen[e / 8]) {
        printf("W=%d %s: chunk (%d, %d) -> element %d not a fresh slot\n", W, IS_K ? "K" : "V",
               r, c, e);
        return false;
      }
      seen[e / 8] = true;
      int rr = -1, cc = -1;
      slot_chunk<W, IS_K>(e / 8, rr, cc);
      if (rr != r || cc != c) {
        printf("W=%d %s: slot %d inverts to (%d, %d), not (%d, %d)\n", W, IS_K ? "K" : "V", e / 8,
               rr, cc, r, c);
        return false;
      }
    }
  return true;
}

template <int W> static bool check_pieces() {
  for (int r = 0; r < 64; ++r) {
    for (int s = 0; s < W / 32; ++s)
      for (int g = 0; g < 4; ++g)
        if (k_step_piece<W>(r, s, g) != lds_chunk<W, true>(r, 4 * s + g)) {
          printf("W=%d: k_step_piece(%d, %d, %d) disagrees\n", W, r, s, g);
          return false;
        }
    if constexpr (W % 64 == 16)
      for (int g = 0; g < 4; ++g)
        if (k_tail16_piece<W>(r, g) !=
            lds_chunk<W, true>(r, 8 * (W / 64) + (g >> 1)) + 4 * (g & 1)) {
          printf("W=%d: k_tail16_piece(%d, %d) disagrees\n", W, r, g);
          return false;
        }
    for (int d = 0; d < W / 16; ++d)
      for (int q4 = 0; q4 < 4; ++q4)
        if (v_piece<W>(r, d, q4) != lds_chunk<W, false>(r, 2 * d + (q4 >> 1)) + 4 * (q4 & 1)) {
          printf("W=%d: v_piece(%d, %d, %d) disagrees\n", W, r, d, q4);
          return false;
        }
  }
  return true;
}

// Largest count of one bank among the 16-byte (or 8-byte) units `u` of a pass.
static int worst_bank(const int* u, int n, int unit_bytes) {
  int count[64] = {}, worst = 0;
  for (int i = 0; i < n; ++i) {
    const int bank = (u[i] * unit_bytes / 4) % 64;
    // every bank the access covers
    for (int k = 0; k < unit_bytes / 4; ++k) {
      const int c = ++count[(bank + k) % 64];
      worst = c > worst ? c : worst;
    }
  }
  return worst;
}

template <int W> static void model(int& k128, int& ktail, int& vtr) {
  k128 = ktail = vtr = 1;
  for (int kb = 0; kb < 4; ++kb)
    for (int s = 0; s < W / 32; ++s)
      for (int g = 0; g < 4; ++g)
        for (int half = 0; half < 2; ++half) {
          int u[8];
          for (int m = 0; m < 8; ++m) u[m] = k_step_piece<W>(key_of(kb, 8 * half + m), s, g) / 8;
          const int w = worst_bank(u, 8, 16);
          k128 = w > k128 ? w : k128;
        }
  if constexpr (W % 64 == 16)
    for (int kb = 0; kb < 4; ++kb)
      for (int gp = 0; gp < 4; gp += 2) {
        int u[32];
        for (int i = 0; i < 32; ++i) u[i] = k_tail16_piece<W>(key_of(kb, i & 15), gp + (i >> 4)) / 4;
        const int w = worst_bank(u, 32, 8);
        ktail = w > ktail ? w : ktail;
      }
  for (int d = 0; d < W / 16; ++d)
    for (int j = 0; j < 2; ++j)
      for (int t = 0; t < 2; ++t)
        for (int gp = 0; gp < 4; gp += 2) {
          int u[32];
          for (int i = 0; i < 32; ++i) {
            const int g = gp + (i >> 4), c16 = i & 15;
            u[i] = v_piece<W>(32 * j + 8 * g + 4 * t + (c16 >> 2), d, c16 & 3) / 4;
          }
          const int w = worst_bank(u, 32, 8);
          vtr = w > vtr ? w : vtr;
        }
}

template <int W> static bool check_width() {
  int k128, ktail, vtr;
  model<W>(k128, ktail, vtr);
  printf("model W=%d k_b128=%d k_tail=%d v_tr=%d\n", W, k128, ktail, vtr);
  return check_layout<W, true>() && check_layout<W, false>() && check_pieces<W>();
}

// The copies keep per-lane offsets for CopyShape::PERIOD rounds only and
// reach round u through a uniform row offset: for every thread and round, the
// chunk the thread copies in round u must be that of round u % PERIOD, in the
// row (u - u % PERIOD) * RPR further on.
template <int W, int BN, int NT, bool IS_K> static bool check_rounds() {
  using CS = CopyShape<W, BN, NT>;
  for (int t = 0; t < NT; ++t)
    for (int u = 0; u < CS::ROUNDS; ++u) {
      const int p = u * NT + t, p0 = (u % CS::PERIOD) * NT + t;
      if (p >= CS::SLOTS) continue;
      int r, c, r0, c0;
      slot_chunk<W, IS_K>(p, r, c);
      slot_chunk<W, IS_K>(p0, r0, c0);
      if (c != c0 || r != r0 + (u - u % CS::PERIOD) * CS::RPR) {
        printf("W=%d BN=%d NT=%d %s: round %d of thread %d is not round %d shifted\n", W, BN,
               NT, IS_K ? "K" : "V", u, t, u % CS::PERIOD);
        return false;
      }
    }
  return true;
}

template <int W, int BN, int NT> static bool check_rounds_kv() {
  printf("rounds W=%d BN=%d NT=%d: %d rounds, %d kept\n", W, BN, NT, CopyShape<W, BN, NT>::ROUNDS,
         CopyShape<W, BN, NT>::PERIOD);
  return check_rounds<W, BN, NT, true>() && check_rounds<W, BN, NT, false>();
}

int main() {
  const bool ok = check_width<64>() && check_width<80>() && check_width<96>() &&
                  check_width<128>() && check_width<192>() && check_width<256>() &&
                  check_rounds_kv<64, 64, 256>() && check_rounds_kv<64, 64, 512>() &&
                  check_rounds_kv<64, 32, 256>() && check_rounds_kv<128, 64, 256>() &&
                  check_rounds_kv<128, 64, 512>() && check_rounds_kv<128, 32, 512>() &&
                  check_rounds_kv<256, 64, 512>() && check_rounds_kv<256, 32, 512>() &&
                  check_rounds_kv<256, 64, 256>() && check_rounds_kv<256, 32, 256>() &&
                  check_rounds_kv<80, 64, 512>() && check_rounds_kv<96, 64, 512>() &&
                  check_rounds_kv<192, 64, 512>();
  printf(ok ? "ok\n" : "FAILED\n");
  return ok ? 0 : 1;
}
