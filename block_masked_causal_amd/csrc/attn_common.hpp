// Device helpers shared by the two-stream attention kernels (forward and
// backward) for gfx950: the MARS mask in interval form, the XOR layouts of
// K/V tiles in LDS, the transposing LDS read and half-wave reductions.
//
// The mask is the 2L x 2L matrix M of the papernotes.org notes on "MARS:
// Enabling Autoregressive Models Multi-Token Generation", key design 1
// (关键设计 1), equation M_ij, over z = [x; x~] with beta(t) = ceil(t/B).
#pragma once

#include "mars_common.hpp"

namespace mars {

// Visible keys of row a: c < hi1, or lo2 <= c < hi2.
__device__ __forceinline__ void row_intervals(int a, int L, int B, int mode, int& hi1, int& lo2,
                                              int& hi2) {
  if (mode == 1 || a < L) {
    hi1 = a + 1;
    lo2 = 0;
    hi2 = 0;
    return;
  }
  const int bb = ((a - L) / B) * B;
  hi1 = bb;
  lo2 = L + bb;
  hi2 = a + 1;
}

// Key ranges a block of query rows [a0, a_last] needs: r1 = [0, r1_hi) and
// r2 = [r2_lo, r2_hi); keys below full_below are visible to every row.
__device__ __forceinline__ void rows_key_ranges(int a0, int a_last, int L, int B, int mode,
                                                int& r1_hi, int& r2_lo, int& r2_hi,
                                                int& full_below) {
  r2_lo = 0;
  r2_hi = 0;
  if (mode == 1 || a_last < L) {
    r1_hi = a_last + 1;
    full_below = a0 + 1;          // causal: fully visible iff every key <= a0
  } else if (a0 >= L) {
    const int t0 = a0 - L, t1 = a_last - L;
    r1_hi = (t1 / B) * B;         // clean keys of strictly earlier blocks
    full_below = (t0 / B) * B;
    r2_lo = L + full_below;       // mask keys of the blocks these rows sit in
    r2_hi = a_last + 1;
  } else {
    r1_hi = a_last + 1;           // rows straddle the stream boundary: test every key
    full_below = 0;
  }
}

// Query rows that see key c: [lo1, hi1) and [lo2, hi2) (the mirror image of
// row_intervals). A clean key is seen by the clean rows from itself on and,
// under the MARS mask, by the mask rows of strictly later blocks; a mask key
// by the mask rows of its own block from itself on.
__device__ __forceinline__ void key_rows(int c, int L, int B, int mode, int& lo1, int& hi1,
                                         int& lo2, int& hi2) {
  const int twoL = 2 * L;
  lo2 = 0;
  hi2 = 0;
  lo1 = c;
  if (mode == 1) {
    hi1 = twoL;
  } else if (c < L) {
    hi1 = L;
    lo2 = min(twoL, L + (c / B + 1) * B);
    hi2 = twoL;
  } else {
    hi1 = min(twoL, L + ((c - L) / B + 1) * B);
  }
}

// K and V tiles sit in LDS unpadded (a direct global->LDS load writes 1 KiB
// contiguously per wave), with the 16-byte chunks of each row permuted by an
// XOR of the row so that the reads below hit all 64 banks:
//  * K rows are read 16 at a time at one chunk (ds_read_b128);
//  * V is read through ds_read_b64_tr_b16, 4 rows x 4 chunks per 32 lanes.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 64 ? (r >> 1) & 7 : r & 15;
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 64 ? ((r >> 1) & 1) << 2 : (r & 3) << 2;
}

// Tiles read both ways (the backward's K, Q and dO tiles: rows for one
// product, transposed for another) use one permutation that keeps both read
// patterns on all 64 banks: the bit reversal of the row's index into swz_k's
// range. swz_k alone leaves the transposing reads 2-way (d = 64) or 4-way
// (d = 128) conflicted, and swz_v leaves the row reads 4-way conflicted.
template <int D>
__device__ __forceinline__ int swz_b(int r) {
  if (D == 64) {
    const int x = (r >> 1) & 7;
    return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1);
  }
  const int x = r & 15;
  return ((x & 1) << 3) | ((x & 2) << 1) | ((x >> 1) & 2) | ((x >> 3) & 1);
}

constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, one L2 each



// Bits [lo, hi) of a 32-bit mask, the range clamped to [0, 32): a lane's
// visible keys among the 32 keys of a tile half (bit t = key t past the
// lane's first key).
__device__ __forceinline__ uint32_t row_bits(int lo, int hi) {
  lo = max(lo, 0);
  hi = min(hi, 32);
  if (hi <= lo) return 0u;
  const uint32_t upto_hi = hi >= 32 ? 0xFFFFFFFFu : (1u << hi) - 1u;
  return upto_hi & ~((1u << lo) - 1u);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// 4 keys x 1 column of a row-major LDS tile (see the lane mapping above)
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16_t* p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p));
}

// max / sum of a value over the two halves of the wave (lanes l and l ^ 32)
__device__ __forceinline__ float halves_max(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

// Heads per workgroup: the largest divisor of the GQA group size that is <= 8.
inline int heads_per_wg(int group) {
  for (int d = 8; d > 1; --d)
    if (group % d == 0) return d;
  return 1;
}

}  // namespace mars
