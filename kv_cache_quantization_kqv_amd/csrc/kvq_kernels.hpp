// kvq_kernels.hpp -- gfx950 (CDNA4) kernels of libkvq, templated on the head
// dimension D and the per-side code widths.  Included once per D by
// kvq_d{16,32,64,128}.hip, which instantiate the dispatchers.
//
// Floating-point contract of the encoder: fp32, round to nearest even, no
// contraction (pragma below and -ffp-contract=off), correctly rounded sqrtf and
// division (-fhip-fp32-correctly-rounded-divide-sqrt).  The butterfly runs its
// stages in ascending order and sums of squares pair adjacent elements level
// by level, so codes, norms and sign bits are reproducible bit for bit.
#pragma once
#pragma clang fp contract(off)

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <utility>

#include "kvq_internal.hpp"

namespace kvq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// bfloat16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// binary16, round to nearest even, overflow to infinity (v_cvt_f16_f32).  The
// argument is pinned in a register first: otherwise the compiler may fuse a
// preceding fp32 multiply into v_fma_mixlo_f16, which rounds once instead of
// fp32-then-fp16 and can differ by one binary16 ulp.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  asm volatile("" : "+v"(f));
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// In-register Sylvester WHT, stages h = 1, 2, 4, ... (ascending).
template <int D>
__device__ __forceinline__ void wht_inplace(float *y) {
#pragma unroll
  for (int h = 1; h < D; h <<= 1) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      if ((i & h) == 0) {
        const float p = y[i], q = y[i + h];
        y[i] = p + q;
        y[i + h] = p - q;
      }
    }
  }
}

// Squares rounded to fp32, summed by adjacent pairs level by level.  The same
// binary tree is evaluated depth first (left half, right half, then their sum),
// which gives identical results with O(log D) live temporaries.
template <int N>
__device__ __forceinline__ float pairwise_sumsq_rec(const float *y) {
  if constexpr (N == 1) {
    return y[0] * y[0];
  } else {
    const float l = pairwise_sumsq_rec<N / 2>(y);
    const float r = pairwise_sumsq_rec<N / 2>(y + N / 2);
    return l + r;
  }
}

template <int D>
__device__ __forceinline__ float pairwise_sumsq(const float *y) {
  return pairwise_sumsq_rec<D>(y);
}

// Bucketize ("KVQuant++" thread, "Fast codebook lookup"): the number of sorted
// thresholds strictly below u, by binary search.  Comparisons use the sign of
// the correctly rounded difference t - u (negative exactly when u > t) as an
// all-ones/zero mask, and candidate thresholds are picked with bit selects, so
// the search needs no lane masks, branches or memory lookups.  Thresholds are
// passed as opaque 32-bit patterns held in VGPRs.
__device__ __forceinline__ uint32_t gt_mask(float u, uint32_t t) {
  return (uint32_t)((int32_t)__float_as_uint(__uint_as_float(t) - u) >> 31);
}
__device__ __forceinline__ uint32_t bsel(uint32_t m, uint32_t a, uint32_t b) {
  return (m & a) | (~m & b);
}

template <int BITS>
__device__ __forceinline__ uint32_t bucketize(float u, const uint32_t *T);

template <>
__device__ __forceinline__ uint32_t bucketize<1>(float u, const uint32_t *T) {
  return gt_mask(u, T[0]) & 1u;
}
template <>
__device__ __forceinline__ uint32_t bucketize<2>(float u, const uint32_t *T) {
  const uint32_t m1 = gt_mask(u, T[1]);
  const uint32_t m0 = gt_mask(u, bsel(m1, T[2], T[0]));
  return (m1 & 2u) | (m0 & 1u);
}
template <>
__device__ __forceinline__ uint32_t bucketize<3>(float u, const uint32_t *T) {
  const uint32_t m2 = gt_mask(u, T[3]);
  const uint32_t m1 = gt_mask(u, bsel(m2, T[5], T[1]));
  const uint32_t m0 = gt_mask(u, bsel(m2, bsel(m1, T[6], T[4]), bsel(m1, T[2], T[0])));
  return (m2 & 4u) | (m1 & 2u) | (m0 & 1u);
}
template <>
__device__ __forceinline__ uint32_t bucketize<4>(float u, const uint32_t *T) {
  const uint32_t m3 = gt_mask(u, T[7]);
  const uint32_t m2 = gt_mask(u, bsel(m3, T[11], T[3]));
  const uint32_t m1 = gt_mask(u, bsel(m3, bsel(m2, T[13], T[9]), bsel(m2, T[5], T[1])));
  const uint32_t t0 = bsel(m3, bsel(m2, bsel(m1, T[14], T[12]), bsel(m1, T[10], T[8])),
                           bsel(m2, bsel(m1, T[6], T[4]), bsel(m1, T[2], T[0])));
  const uint32_t m0 = gt_mask(u, t0);
  return (m3 & 8u) | (m2 & 4u) | (m1 & 2u) | (m0 & 1u);
}

// Place code i of a D-vector into the record's little-endian word image.
// Widths 1, 2, 4: bit offset i*w.  Width 3: low two bits in a 2-bit plane
// (bit 2i), high bit in a 1-bit plane starting at byte D/4 (bit 2D + i).
template <int D, int BITS>
__device__ __forceinline__ void place_code(uint32_t *rec, int i, uint32_t code) {
  if constexpr (BITS == 3) {
    rec[(2 * i) >> 5] |= (code & 3u) << ((2 * i) & 31);
    rec[(2 * D + i) >> 5] |= (code >> 2) << ((2 * D + i) & 31);
  } else {
    rec[(i * BITS) >> 5] |= code << ((i * BITS) & 31);
  }
}

// Store NB bytes from a little-endian word image with the widest aligned chunks.
template <int NB>
__device__ __forceinline__ void store_bytes(uint8_t *dst, const uint32_t *w) {
  constexpr int CH = (NB % 16 == 0) ? 16 : (NB % 8 == 0) ? 8 : (NB % 4 == 0) ? 4 : (NB % 2 == 0) ? 2 : 1;
#pragma unroll
  for (int o = 0; o < NB; o += CH) {
    if constexpr (CH == 16) {
      *(u32x4 *)(dst + o) = u32x4{w[o / 4], w[o / 4 + 1], w[o / 4 + 2], w[o / 4 + 3]};
    } else if constexpr (CH == 8) {
      *(u32x2 *)(dst + o) = u32x2{w[o / 4], w[o / 4 + 1]};
    } else if constexpr (CH == 4) {
      *(uint32_t *)(dst + o) = w[o / 4];
    } else if constexpr (CH == 2) {
      *(uint16_t *)(dst + o) = (uint16_t)(w[o / 4] >> (8 * (o % 4)));
    } else {
      dst[o] = (uint8_t)(w[o / 4] >> (8 * (o % 4)));
    }
  }
}

// ---------------------------------------------------------------------------
// Exact bucketize by table ("KVQuant++" thread, "Fast codebook lookup": a
// lookup against sorted thresholds instead of a nearest-centroid search).
// The top 9 + MB bits of u's fp32 pattern (sign, exponent, MB mantissa bits;
// MB = 2 for 4-bit codes, 1 for 3-bit codes) cut the line into cells: a cell
// of non-negative patterns holds [lo, hi], one of negative patterns
// [-hi, -lo], with hi < (1 + 2^-MB) lo (and the cells of prefix 0 reaching
// down to +0 and -0).  Consecutive positive thresholds of the tables used
// here fall in different cells and the smallest is above the prefix-0 cell
// (the host checks this for every table it builds), so a cell holds at most
// one threshold: the entry of a cell is (that threshold or +inf, the number
// of thresholds below the cell), and
//   code = count + (threshold < u)
// equals #{thresholds < u} (ties go to the lower cell; -0 and +0 against the
// zero threshold compare as IEEE floats do).
// ---------------------------------------------------------------------------
// Codes of at most kCmpMaxBits bits are found by compares against the
// thresholds; wider ones through the cell table, except at d = 8, where
// neighbouring thresholds can share a cell (compares for every width).
constexpr int kCmpMaxBits = 2;
template <int BITS, bool CELLS = true>
struct BucketTables {
  static constexpr bool LUT = CELLS && BITS > kCmpMaxBits;
  static constexpr int MB = BITS >= 4 ? 2 : 1;       // mantissa bits of the cell prefix
  static constexpr int SHIFT = 23 - MB;
  static constexpr int NCELL = 1 << (9 + MB);
  f32x2 cell[LUT ? NCELL : 1];  // (threshold inside the cell or +inf, count below as bits)
  float cent[16];
};

template <int BITS, bool CELLS>
__device__ void build_bucket_tables(BucketTables<BITS, CELLS> &bt, const float *thr, const float *cent,
                                    int tid, int nthreads) {
  using BT = BucketTables<BITS, CELLS>;
  constexpr int K = 1 << BITS;
  if constexpr (BT::LUT) {
    for (int i = tid; i < BT::NCELL; i += nthreads) {
      // the cell's range as (lower, upper) end points in the order of floats
      const uint32_t a = (uint32_t)(i & (BT::NCELL / 2 - 1)) << BT::SHIFT;
      const uint32_t b = a | ((1u << BT::SHIFT) - 1u);
      const float m0 = __uint_as_float(a), m1 = __uint_as_float(b);
      const bool neg = i >= BT::NCELL / 2;
      const float lo = neg ? -m1 : m0, hi = neg ? -m0 : m1;
      // thresholds ascend: count those below lo by binary search; the next one
      // is the cell's threshold if it does not exceed hi
      uint32_t below = 0;
#pragma unroll
      for (int step = K / 2; step >= 1; step >>= 1)
        if (below + step <= (uint32_t)(K - 1) && thr[below + step - 1] < lo) below += step;
      const float inside = (below < (uint32_t)(K - 1) && thr[below] <= hi) ? thr[below] : INFINITY;
      bt.cell[i] = f32x2{inside, __uint_as_float(below)};
    }
  }
  if (tid < 16) bt.cent[tid] = cent[tid];
}

template <int BITS>
__device__ __forceinline__ uint32_t bucketize_lut(float u, const BucketTables<BITS, true> &bt) {
  const f32x2 e = bt.cell[__float_as_uint(u) >> BucketTables<BITS, true>::SHIFT];
  return __float_as_uint(e.y) + (e.x < u ? 1u : 0u);
}

// The same count by comparisons against the positive thresholds held in
// scalar registers (for narrow codes, where K/2 - 1 compares cost no more than
// the two table reads).  Bit patterns of non-negative floats order like the
// floats, so  P < |u|  is  bits(P) < bits(|u|)  and  P <= |u|  is
// bits(P) < bits(|u|) + 1;  u <= 0 (both zeros included) takes the second
// form, and its code K/2 - 1 - le is the complement of K/2 + le in BITS bits.
template <int BITS>
__device__ __forceinline__ uint32_t bucketize_cmp(float u, const float *thr) {
  constexpr uint32_t K2 = 1u << (BITS - 1);
  const uint32_t neg = (u <= 0.0f) ? 1u : 0u;
  const uint32_t key = (__float_as_uint(u) & 0x7FFFFFFFu) + neg;
  uint32_t n = K2;
#pragma unroll
  for (uint32_t k = 0; k + 1 < K2; ++k) n += (__float_as_uint(thr[K2 + k]) < key) ? 1u : 0u;
  return n ^ (neg ? 2u * K2 - 1u : 0u);
}

template <int BITS, bool CELLS>
__device__ __forceinline__ uint32_t bucketize_code(float u, const BucketTables<BITS, CELLS> &bt, const float *thr) {
  if constexpr (!BucketTables<BITS, CELLS>::LUT) return bucketize_cmp<BITS>(u, thr);
  else return bucketize_lut<BITS>(u, bt);
}

// y[i] <- y[i] + s * (y[i] of the partner lane, lane ^ 1), for 8 coordinates,
// one v_fmac_f32 with a DPP quad-permute source each: s = +-1 makes the
// product exact, so each result is the one rounding of y[i] +- partner.  The
// leading s_nop gives the DPP reads the two wait states they need after the
// VALU writes that produced y (issued before the block).
__device__ __forceinline__ void fmac_xor1_x8(float *y, float s) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %4, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %5, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %6, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %7, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
      : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3]), "+v"(y[4]), "+v"(y[5]), "+v"(y[6]), "+v"(y[7])
      : "v"(s));
}

// As fmac_xor1_x8 with the partner lane ^ 2.
__device__ __forceinline__ void fmac_xor2_x8(float *y, float s) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %4, %4, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %5, %5, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %6, %6, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %7, %7, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
      : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3]), "+v"(y[4]), "+v"(y[5]), "+v"(y[6]), "+v"(y[7])
      : "v"(s));
}

// Value of the partner lane (lane ^ 2) through a DPP quad permute.
__device__ __forceinline__ float xor2_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// Value of the partner lane (lane ^ 1) through a DPP quad permute (no LDS).
__device__ __forceinline__ float xor1_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t xor1_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}

// Sum over each row of 16 lanes, left in every lane of the row (DPP: partner
// lane ^1, ^2, then the mirrored lane within 8 and within 16).  Depth 4.
__device__ __forceinline__ float row_sum16(float v) {
  v = v + xor1_f(v);
  v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}
// Value of lane l (uniform l).
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Codes of DL consecutive coordinates packed at compile-time positions: widths
// 1, 2, 4 as one little-endian image; width 3 as a 2-bit plane image (DL/16
// words) followed by a 1-bit plane image (DL/32 words, at least one).
template <int DL, int BITS>
struct LocalCodes {
  static constexpr int NA = BITS == 3 ? (2 * DL + 31) / 32 : (DL * BITS + 31) / 32;
  static constexpr int NB = BITS == 3 ? (DL + 31) / 32 : 0;
  uint32_t w[NA + NB];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int k = 0; k < NA + NB; ++k) w[k] = 0u;
  }
  __device__ __forceinline__ void put(int i, uint32_t code) {
    if constexpr (BITS == 3) {
      w[(2 * i) >> 5] |= (code & 3u) << ((2 * i) & 31);
      w[NA + (i >> 5)] |= (code >> 2) << (i & 31);
    } else {
      w[(i * BITS) >> 5] |= code << ((i * BITS) & 31);
    }
  }
};

// Record image of a D-vector from the halves built by a lane pair (LPV = 2):
// own = coordinates [0, DL), other = [DL, 2 DL).  Layout as in place_code.
template <int D, int DL, int BITS, int RECW>
__device__ __forceinline__ void join_halves(uint32_t *rec, const LocalCodes<DL, BITS> &own,
                                            const LocalCodes<DL, BITS> &other) {
  using LC = LocalCodes<DL, BITS>;
  if constexpr (BITS == 3) {
#pragma unroll
    for (int k = 0; k < LC::NA; ++k) {
      rec[k] = own.w[k];
      rec[LC::NA + k] = other.w[k];
    }
#pragma unroll
    for (int k = 0; k < LC::NB; ++k) {
      rec[2 * LC::NA + k] = own.w[LC::NA + k];
      rec[2 * LC::NA + LC::NB + k] = other.w[LC::NA + k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < LC::NA; ++k) {
      rec[k] = own.w[k];
      rec[LC::NA + k] = other.w[k];
    }
  }
}

// One lane's quarter of a d = 256 record (LPV = 4): codes of coordinates
// [DL q, DL q + DL).  Widths 1, 2, 4: bytes [q DL b/8, ...); width 3: bytes
// [q DL/4, ...) of the 2-bit plane and [D/4 + q DL/8, ...) of the 1-bit plane.
template <int D, int DL, int BITS>
__device__ __forceinline__ void store_quarter(uint8_t *rec, const LocalCodes<DL, BITS> &lc, int q) {
  using LC = LocalCodes<DL, BITS>;
  if constexpr (BITS == 3) {
    store_bytes<DL / 4>(rec + q * (DL / 4), lc.w);
    store_bytes<DL / 8>(rec + D / 4 + q * (DL / 8), lc.w + LC::NA);
  } else {
    store_bytes<DL * BITS / 8>(rec + q * (DL * BITS / 8), lc.w);
  }
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Constant-address-space view of a device buffer that every lane reads at the
// same address (the loads become scalar loads).
typedef const __attribute__((address_space(4))) float cfloat;

// ---------------------------------------------------------------------------
// Sketch-side helpers shared by the encoders.  S is staged in LDS with a padded
// row pitch P2 = 2D + 16 bytes; residual rows r~ (bf16) use the same pitch.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void stage_sketch(unsigned char *S_s, const uint16_t *S, int tid) {
  constexpr int P2 = D * 2 + 16;
  for (int i = tid; i < D * (D / 8); i += 256) {     // 16-B chunks of S
    const int r = i / (D / 8), c = i - r * (D / 8);
    *(u32x4 *)(S_s + r * P2 + c * 16) = *(const u32x4 *)(S + (size_t)r * D + c * 8);
  }
}

// Largest sketch row norm (fp32, rounded up), for the sign-certification bound.
template <int D, int SP = D * 2 + 16>
__device__ __forceinline__ float sketch_row_norm_max(const unsigned char *S_s, int lane) {
  constexpr int P2 = SP;
  constexpr int NCT = (D + 31) / 32;
  float mx = 0.0f;
#pragma unroll 1
  for (int ct = 0; ct < NCT; ++ct) {
    const int col = ct * 32 + (lane & 31);
    float sq = 0.0f;
    if (col < D) {
      const uint16_t *sr = (const uint16_t *)(S_s + col * P2);
      for (int i = 0; i < D; ++i) {
        const float v = bf16_to_f32(sr[i]);
        sq = sq + v * v;
      }
    }
    mx = fmaxf(mx, sqrtf(sq) * (1.0f + 0x1p-12f));
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  return mx;
}

// Sign bits of z = S r~ for the residual rows of one wave's tile (NRT blocks of
// 32 rows at `stage`, pitch P2), written to signs + (slot0 + t) * D/8 for the
// valid rows t < nvalid.  rn_s[t] holds D 2^-22 (1 + 2^-7) ||r_t||.
//
// z^T = S r~^T per 32-token block with v_mfma_f32_32x32x16_bf16: A = S rows
// (sketch rows k), B = r~ rows (tokens t).  Output register j of lane l is
// z[k][t] with k = 32 ct + 8 (j/4) + 4 (l/32) + (j%4) and t = l%32, so a lane
// holds 16 of its token's sign bits per 32-row block and lane l^32 the other
// 16.  A sign is taken from z when |z| exceeds a bound on the accumulation
// error of any summation order, D * 2^-22 * ||S_k|| * ||r~|| (+2^-100 for
// flushed denormals); the rest are settled exactly (below).
}  // namespace kvq

#include "kvq_vgroup.hpp"

namespace kvq {

// Rows rlo <= t < nvalid of the tile are tokens; their sign records go to
// signs_out at slot0 + t, or (TO_LDS, d = 128) to srows + SP t in LDS.  S_s:
// the sketch rows, SPITCH bytes apart (staged in LDS, or in memory at d =
// 256); the stage holds VTR rows (a 32-row block past them reads as zero).
// Below d = 16 (one sketch MFMA step would exceed the row) every sign is the
// ascending fp64 sum itself, one token per lane.
template <int D, int NRT, bool TO_LDS = false, int SP = 16, int SPITCH = D * 2 + 16,
          int VTR = 32 * NRT>
__device__ __forceinline__ void sketch_signs(const unsigned char *stage, const unsigned char *S_s,
                                             const float *rn_s, float a_snmax, int rlo, int nvalid,
                                             size_t slot0, uint8_t *signs_out, uint8_t *srows,
                                             int lane) {
  constexpr int P2 = D * 2 + 16;
  constexpr int NCT = (D + 31) / 32;
  if constexpr (D < 16) {
    static_assert(!TO_LDS && D % 8 == 0, "direct signs: per-slot records of whole bytes");
#pragma unroll 1
    for (int t = lane; t < VTR; t += 64) {
      if (t < rlo || t >= nvalid) continue;
      const uint16_t *rr = (const uint16_t *)(stage + t * P2);
      uint8_t *dst = signs_out + (slot0 + (size_t)t) * (D / 8);
#pragma unroll
      for (int kb = 0; kb < D / 8; ++kb) {
        uint32_t by = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint16_t *sr = (const uint16_t *)(S_s + (8 * kb + e) * SPITCH);
          double sum = 0.0;
          for (int i = 0; i < D; ++i)
            sum = sum + (double)bf16_to_f32(sr[i]) * (double)bf16_to_f32(rr[i]);
          by |= (sum >= 0.0 ? 1u : 0u) << e;
        }
        dst[kb] = (uint8_t)by;
      }
    }
    return;
  }
#pragma unroll 1
  for (int rt = 0; rt < NRT; ++rt) {
    const int t = rt * 32 + (lane & 31);                  // token row in the tile
    const bool tin = t < VTR;
    const float rbt = tin ? rn_s[t] : 0.0f;
    // B operands (this block's residual rows), read once for all row blocks
    u32x4 rv[D >= 16 ? D / 16 : 1];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      rv[ks] = tin ? *(const u32x4 *)(stage + t * P2 + (ks * 16 + 8 * (lane >> 5)) * 2)
                   : u32x4{0u, 0u, 0u, 0u};
    uint32_t sgw[NCT];
#pragma unroll 1
    for (int ct = 0; ct < NCT; ++ct) {
      f32x16 acc;
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
      const int krow = ct * 32 + (lane & 31);             // A row of this lane
      const bool kok = krow < D;
      const int ks_row = kok ? krow : 0;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int k0 = ks * 16 + 8 * (lane >> 5);
        u32x4 sv = *(const u32x4 *)(S_s + ks_row * SPITCH + k0 * 2);
        if (!kok) sv = u32x4{0u, 0u, 0u, 0u};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, sv),
                                                      __builtin_bit_cast(bf16x8, rv[ks]), acc,
                                                      0, 0, 0);
      }
      // certified signs
      const float bound = fmaf(a_snmax, rbt, 0x1p-100f);
      uint32_t unsure = 0u;
      float zmin = INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) zmin = fminf(zmin, fabsf(acc[j]));
      // bit 8 (j >> 2) + 4 (lane >> 5) + (j & 3) = sketch row % 32 of entry j.
      // Where |z| > bound (> 0), z > 0 is exactly "sign bit clear": the sign
      // bits enter one funnel shift each (v_alignbit), highest position
      // first, with four zero bits between the groups of four; the other
      // entries are settled below.
      uint32_t neg = 0u;
#pragma unroll
      for (int g = 3; g >= 0; --g) {
        if (g < 3) neg <<= 4;
#pragma unroll
        for (int e = 3; e >= 0; --e)
          neg = __builtin_amdgcn_alignbit(neg, __float_as_uint(acc[4 * g + e]), 31);
      }
      uint32_t bits = (~neg & 0x0F0F0F0Fu) << (4 * (lane >> 5));
      // the per-bit mask only where some entry of the wave is uncertain (rare);
      // !(zmin > bound) also catches NaN
      const bool trow = tin && t >= rlo && t < nvalid;
      if (__ballot(!(zmin > bound) && trow)) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int bp = 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
          unsure |= (!(fabsf(acc[j]) > bound) ? 1u : 0u) << bp;
        }
      }
      if constexpr (D < 32) unsure &= (1u << D) - 1u;                 // rows >= D do not exist
      if (!trow) unsure = 0u;                                          // padding rows of the tile
      // Uncertain entries, one (lane, row) at a time for the whole wave.  The
      // products s_i r~_i of two bf16 values are exact in fp32 (16-bit
      // significands; |s r~| >= 2^-126 unless tiny, covered by 2^-110
      // below).  The lanes sum them in a tree of depth <= 9 (d <= 256), so
      // the sum T is within 9 2^-24 A of the exact sum E (A = sum |s_i r~_i|),
      // and the oracle's ascending fp64 sum is within 255 2^-53 A of E: beyond
      // 2^-20 A + 2^-110 the signs of all three agree.  Otherwise (E = 0
      // included) the ascending fp64 sum itself is formed, by every lane
      // alike from uniform addresses.
      uint64_t pend = __ballot(unsure != 0u);
      while (pend) {
        const int src = __builtin_ctzll(pend);
        const uint32_t um = (uint32_t)__builtin_amdgcn_readlane((int)unsure, src);
        const int bp = __builtin_ctz(um);
        const int k = ct * 32 + bp;
        const unsigned char *rr = stage + (rt * 32 + (src & 31)) * P2;
        const unsigned char *sr = S_s + k * SPITCH;
        float ps = 0.0f, pa = 0.0f;
        if constexpr (D >= 128) {
          // two products per dword, D / 128 dwords per lane
#pragma unroll
          for (int c = 0; c < D / 128; ++c) {
            const uint32_t sw = *(const uint32_t *)(sr + 4 * (lane + 64 * c));
            const uint32_t rw = *(const uint32_t *)(rr + 4 * (lane + 64 * c));
            const float p0 = bf16_lo(sw) * bf16_lo(rw), p1 = bf16_hi(sw) * bf16_hi(rw);
            ps = ps + (p0 + p1);
            pa = pa + (fabsf(p0) + fabsf(p1));
          }
        } else {
          if (lane < D) {
            const float p = bf16_to_f32(*(const uint16_t *)(sr + 2 * lane)) *
                            bf16_to_f32(*(const uint16_t *)(rr + 2 * lane));
            ps = p;
            pa = fabsf(p);
          }
        }
        ps = row_sum16(ps);
        pa = row_sum16(pa);
        const float T = (lane_f(ps, 0) + lane_f(ps, 16)) + (lane_f(ps, 32) + lane_f(ps, 48));
        const float A = (lane_f(pa, 0) + lane_f(pa, 16)) + (lane_f(pa, 32) + lane_f(pa, 48));
        uint32_t bit;
        if (fabsf(T) > fmaf(A, 0x1p-20f, 0x1p-110f)) {
          bit = T > 0.0f ? 1u : 0u;
        } else {
          double sum = 0.0;
          for (int i = 0; i < D; ++i)
            sum = sum + (double)bf16_to_f32(*(const uint16_t *)(sr + 2 * i)) *
                            (double)bf16_to_f32(*(const uint16_t *)(rr + 2 * i));
          bit = sum >= 0.0 ? 1u : 0u;
        }
        if (lane == src) {
          bits = (bits & ~(1u << bp)) | (bit << bp);
          unsure &= unsure - 1u;
        }
        pend = __ballot(unsure != 0u);
      }
      sgw[ct] = bits | (uint32_t)__shfl_xor((int)bits, 32, 64);
    }
    const bool tvalid = tin && t >= rlo && t < nvalid && lane < 32;
    if constexpr (TO_LDS) {
      static_assert(D == 128, "LDS sign rows exist at d = 128 only");
      if (lane < 32) *(u32x4 *)(srows + SP * t) = u32x4{sgw[0], sgw[1], sgw[2], sgw[3]};
    } else if (tvalid) {
      const size_t tslot = slot0 + (size_t)t;
      uint8_t *dst = signs_out + tslot * (D / 8);
      if constexpr (D == 256) {
        *(u32x4 *)dst = u32x4{sgw[0], sgw[1], sgw[2], sgw[3]};
        *(u32x4 *)(dst + 16) = u32x4{sgw[4], sgw[5], sgw[6], sgw[7]};
      } else if constexpr (D == 128) {
        *(u32x4 *)dst = u32x4{sgw[0], sgw[1], sgw[2], sgw[3]};
      } else if constexpr (D == 64) {
        *(u32x2 *)dst = u32x2{sgw[0], sgw[1]};
      } else if constexpr (D == 32) {
        *(uint32_t *)dst = sgw[0];
      } else {
        *(uint16_t *)dst = (uint16_t)(sgw[0] & 0xFFFFu);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Quantize-on-write.  Blocks of 4 waves share the bucketize tables and (sketch
// sides) the sketch matrix S, staged once in LDS with a padded row pitch; each
// wave then walks its own tiles.  A tile is VT consecutive tokens of one
// (b, h), each token owned by LPV lanes (LPV = 2 for D = 128, else 1), each
// lane holding DL = D/LPV consecutive coordinates in registers.  The tile is
// read with coalesced 16-B loads into a padded LDS stage; the next tile's loads
// are issued before the current one is processed.
// RK: none, Walsh-Hadamard, or randomized Hadamard (coordinate signs flipped
// first; a flip is exact).  Butterfly stages h < DL run in registers; the last
// stage of a split vector is one exchange with the partner lane (lane ^ 1),
// and the pairwise sum of squares of a split vector is (left half sum) + (right
// half sum), which is the root of the same adjacent-pair tree.  Then
// u = y * (1/nu), bucketize, pack.  Sketch sides write the bf16 residual
// halves back to the stage and take the signs of S r~ (sketch_signs).
// Tiles are aligned to VT cache slots (the first one may start before t0, the
// last end after t0 + T; those rows are padding).  VG: value side at d = 128
// in token groups; the codes go to LDS as one nibble per coordinate and the
// sign records to LDS, and the wave then writes whole groups (vg_emit_*).
// ---------------------------------------------------------------------------
// At d = 256 a lane holds 64 coordinates and the encoder does not fit two
// blocks per CU: one block per CU lets it use the whole register file (spills
// go to accumulator registers rather than scratch memory).
template <int D, int BITS, int RK, bool QJL, bool BF16, bool VG>
__global__ __launch_bounds__(256, D > 128 ? 1 : 2)
void quantize_kernel(const QuantArgs a) {
  constexpr int LPV = D > 128 ? 4 : (D > 64 ? 2 : 1);   // lanes per vector
  constexpr int DL = D / LPV;                // coordinates per lane
  constexpr int VT = 64 / LPV;               // vectors per tile
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int ROWB = D * ESZ;
  constexpr int PITCH = ROWB + 16;
  constexpr int CPR = ROWB / 16;             // 16-B chunks per row
  constexpr int NLD = VT * CPR / 64;         // chunks per lane
  constexpr int RECB = D * BITS / 8;
  constexpr int RECW = (RECB + 3) / 4;
  constexpr int NRT = VT >= 32 ? VT / 32 : 1;   // 32-row sketch blocks (16 valid rows at d = 256)
  constexpr int P2 = D * 2 + 16;             // bf16 row pitch (residuals, S)
  // S staged in LDS with pitch P2, or at d = 256 (where it would not fit
  // beside the tiles) read from memory, rows 2 d bytes apart
  constexpr bool SMEM = D > 128;
  constexpr int SPITCH = SMEM ? 2 * D : P2;
  constexpr int SBYTES = (QJL && !SMEM) ? D * P2 : 16;
  static_assert(VT * P2 <= VT * PITCH, "residual rows must fit the staging buffer");
  static_assert((VT * CPR) % 64 == 0, "tile copy must split evenly over the wave");
  __shared__ __attribute__((aligned(16))) unsigned char stage_all[4][VT * PITCH];
  __shared__ __attribute__((aligned(16))) unsigned char S_s[SBYTES];
  __shared__ BucketTables<BITS, (D >= 16)> bt;
  __shared__ float rn_all[4][VT];
  static_assert(!VG || D == 128, "token groups exist at d = 128 only");
  // VG: once the stage's residual rows are consumed, row t of the stage (pitch
  // P2) holds slot t's per-slot code record in bytes [0, RECB) and its sign
  // record in the row's padding, bytes [2D, 2D + 16)
  static_assert(!VG || (RECB <= 2 * D && VT * P2 <= VT * PITCH), "group rows must fit the stage");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned char *stage = stage_all[wave];
  float *rn_s = rn_all[wave];
  const int vrow = lane / LPV;               // token row of this lane in the tile
  const int lead = a.t0 % VT;                // padding rows before t0 in the first tile
  const int half = lane % LPV;               // which part of the vector (coordinates half*DL ...)
  build_bucket_tables(bt, a.thr, a.cent, tid, 256);
  if constexpr (QJL && !SMEM) stage_sketch<D>(S_s, a.S, tid);
  __syncthreads();
  const unsigned char *Ssrc = SMEM ? (const unsigned char *)a.S : S_s;
  float a_snmax = 0.0f;
  if constexpr (QJL) a_snmax = sketch_row_norm_max<D, SPITCH>(Ssrc, lane);
  // randomized Hadamard: this lane's sign words (coordinates half*DL ...)
  constexpr int NMW = (DL + 31) / 32;
  uint32_t mw[NMW];
#pragma unroll
  for (int w = 0; w < NMW; ++w) {
    mw[w] = 0u;
    if constexpr (RK == RK_RHT) mw[w] = a.rsign[half * NMW + w];
  }

  const int tile0 = blockIdx.x * 4 + wave;
  const int tstride = gridDim.x * 4;
  u32x4 pf[NLD];
  auto fetch = [&](int tile) {
    const int bh = tile / a.tiles_per_bh;
    const int tt = tile - bh * a.tiles_per_bh;
    const int b = bh / a.H, h = bh - b * a.H;
    const int tbase = tt * VT - lead;
    const int rlo = max(0, -tbase), nvalid = min(VT, a.T - tbase);
    // chunk lane + 64k is row lane/CPR + (64/CPR) k, column lane%CPR: one base
    // pointer per lane and a fixed row step (few live registers across the loop)
    const long long rstride = a.st * ESZ;
    const unsigned char *src = (const unsigned char *)a.src +
        ((long long)b * a.sb + (long long)h * a.sh + (long long)tbase * a.st) * ESZ +
        (lane / CPR) * rstride + (lane % CPR) * 16;
    const long long kstep = (64 / CPR) * rstride;
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int r = lane / CPR + (64 / CPR) * k;
      pf[k] = u32x4{0u, 0u, 0u, 0u};
      if (r >= rlo && r < nvalid) pf[k] = *(const u32x4 *)(src + k * kstep);
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int ci = lane + 64 * k;
      const int r = ci / CPR, cc = ci - r * CPR;
      *(u32x4 *)(stage + r * PITCH + cc * 16) = pf[k];
    }
  };
  if (tile0 < a.total_tiles) {
    fetch(tile0);
    stash();
  }
  wave_sync();

#pragma unroll 1
  for (int tile = tile0; tile < a.total_tiles; tile += tstride) {
    const int bh = tile / a.tiles_per_bh;
    const int tt = tile - bh * a.tiles_per_bh;
    const int tbase = tt * VT - lead;
    const int rlo = max(0, -tbase), nvalid = min(VT, a.T - tbase);

    float y[DL];
    const unsigned char *myrow = stage + vrow * PITCH + half * DL * ESZ;
    if constexpr (BF16) {
#pragma unroll
      for (int c = 0; c < DL / 8; ++c) {
        const u32x4 v = *(const u32x4 *)(myrow + c * 16);
        y[8 * c + 0] = bf16_lo(v.x); y[8 * c + 1] = bf16_hi(v.x);
        y[8 * c + 2] = bf16_lo(v.y); y[8 * c + 3] = bf16_hi(v.y);
        y[8 * c + 4] = bf16_lo(v.z); y[8 * c + 5] = bf16_hi(v.z);
        y[8 * c + 6] = bf16_lo(v.w); y[8 * c + 7] = bf16_hi(v.w);
      }
    } else {
#pragma unroll
      for (int c = 0; c < DL / 4; ++c) {
        const u32x4 v = *(const u32x4 *)(myrow + c * 16);
        y[4 * c + 0] = __uint_as_float(v.x); y[4 * c + 1] = __uint_as_float(v.y);
        y[4 * c + 2] = __uint_as_float(v.z); y[4 * c + 3] = __uint_as_float(v.w);
      }
    }
    wave_sync();
    const int next = tile + tstride;
    // prefetch the next tile now, or (sketched sides) once the coordinates are
    // dead, so the prefetch registers overlap the sketch products instead
    if constexpr (!QJL) {
      if (next < a.total_tiles) fetch(next);
    }

    if constexpr (RK == RK_RHT) {
      // passed through an asm tied to the tile: otherwise all DL sign masks
      // are hoisted out of the tile loop and stay live (register spills)
      uint32_t m[NMW];
#pragma unroll
      for (int w = 0; w < NMW; ++w) {
        m[w] = mw[w];
        asm("" : "+v"(m[w]) : "v"(tile));
      }
#pragma unroll
      for (int i = 0; i < DL; ++i)
        y[i] = __uint_as_float(__float_as_uint(y[i]) ^ ((m[i >> 5] << (31 - (i & 31))) & 0x80000000u));
    }
    // sign of this lane's coordinates as held (see the last butterfly stage)
    float held = 1.0f;
    if constexpr (RK != RK_NONE) {
      wht_inplace<DL>(y);
      if constexpr (LPV >= 2) {
        // stage h = DL: (y_i, y_{i+DL}) -> (y_i + y_{i+DL}, y_i - y_{i+DL}).  The
        // lower lane forms own + partner; the upper lane own - partner, the
        // exact negation of the rounded difference, and keeps that sign until
        // the scaling below (the squares do not see it).
        held = (half & 1) ? -1.0f : 1.0f;
        static_assert(DL % 8 == 0, "butterfly stage in groups of 8");
#pragma unroll
        for (int i = 0; i < DL; i += 8) fmac_xor1_x8(y + i, held);
      }
      if constexpr (LPV == 4) {
        // stage h = 2 DL between lanes q and q ^ 2, which hold the same sign:
        // own +- partner is that sign times the true sum / the negated
        // difference
        const float s2 = (half & 2) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < DL; i += 8) fmac_xor2_x8(y + i, s2);
        held *= s2;
      }
    }
    float ss = pairwise_sumsq<DL>(y);
    // the adjacent-pair tree over the lanes of the vector (lower part first)
    if constexpr (LPV >= 2) {
      const float o = xor1_f(ss);
      ss = (half & 1) ? (o + ss) : (ss + o);
    }
    if constexpr (LPV == 4) {
      const float o = xor2_f(ss);
      ss = (half & 2) ? (o + ss) : (ss + o);
    }
    const float nu = sqrtf(ss);
    // u = y * (1/nu) with the held sign folded in (a negation is exact)
    const float rcp = nu == 0.0f ? 0.0f : held * (1.0f / nu);
    // codes: the record layout (per-slot records), or one nibble per
    // coordinate (token groups: the regrouping reads nibbles)
    LocalCodes<DL, BITS> lc;
    lc.clear();
    uint32_t nib[VG ? DL / 8 : 1] = {};
#pragma unroll
    for (int i = 0; i < DL; ++i) {
      const float u = y[i] * rcp;
      const uint32_t code = bucketize_code<BITS>(u, bt, a.thr);
      if constexpr (VG) nib[i >> 3] |= code << (4 * (i & 7));
      else lc.put(i, code);
      if constexpr (QJL) y[i] = u - bt.cent[code];
      // keep at most 16 coordinates' table lookups in flight (register pressure)
      if ((i & 15) == 15) __builtin_amdgcn_sched_barrier(0);
    }
    const bool valid = vrow >= rlo && vrow < nvalid;
    const size_t slot = (size_t)bh * a.cap + (size_t)(a.t0 + tbase + vrow);
    uint32_t rec[RECW];
    if constexpr (VG) {
      // the nibbles stay in registers until the stage is free (below); packed
      // here, or the compiler defers the packing and keeps every code live
#pragma unroll
      for (int k = 0; k < DL / 8; ++k) asm volatile("" : "+v"(nib[k]));
    } else if constexpr (LPV == 4) {
      // each lane writes its quarter of the record itself (below)
    } else if constexpr (LPV == 2) {
      // each lane packed its own half; the lower lane joins the two images
      LocalCodes<DL, BITS> oth;
#pragma unroll
      for (int k = 0; k < LocalCodes<DL, BITS>::NA + LocalCodes<DL, BITS>::NB; ++k)
        oth.w[k] = xor1_u(lc.w[k]);
      join_halves<D, DL, BITS, RECW>(rec, lc, oth);
    } else if constexpr (BITS == 3 && D == 8) {
      // 2-bit plane (2 bytes), then the 1-bit plane (1 byte)
      rec[0] = (lc.w[0] & 0xFFFFu) | (lc.w[1] << 16);
    } else {
#pragma unroll
      for (int k = 0; k < RECW; ++k) rec[k] = 0u;
#pragma unroll
      for (int k = 0; k < LocalCodes<DL, BITS>::NA; ++k) rec[k] = lc.w[k];
      if constexpr (BITS == 3) {
#pragma unroll
        for (int k = 0; k < LocalCodes<DL, BITS>::NB; ++k)
          rec[LocalCodes<DL, BITS>::NA + k] |= lc.w[LocalCodes<DL, BITS>::NA + k];
      }
    }
    if constexpr (LPV == 4) {
      if (valid) store_quarter<D, DL, BITS>(a.codes + slot * RECB, lc, half);
    }
    if (valid && half == 0) {
      if constexpr (!VG && LPV < 4) store_bytes<RECB>(a.codes + slot * RECB, rec);
      a.norm[slot] = f32_to_f16_bits(nu * a.scale);
    }

    if constexpr (QJL) {
      float rs = pairwise_sumsq<DL>(y);
      if constexpr (LPV >= 2) {
        const float o = xor1_f(rs);
        rs = (half & 1) ? (o + rs) : (rs + o);
      }
      if constexpr (LPV == 4) {
        const float o = xor2_f(rs);
        rs = (half & 2) ? (o + rs) : (rs + o);
      }
      const float rho = sqrtf(rs);
      if (valid && half == 0) a.rnorm[slot] = f32_to_f16_bits(rho);
      // bf16 residual halves into the stage (hardware round-to-nearest-even pack)
      unsigned char *rrow = stage + vrow * P2 + half * DL * 2;
#pragma unroll
      for (int c = 0; c < DL / 8; ++c) {
        uint32_t wv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f32x2 pr = {y[8 * c + 2 * k], y[8 * c + 2 * k + 1]};
          wv[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
        }
        *(u32x4 *)(rrow + c * 16) = u32x4{wv[0], wv[1], wv[2], wv[3]};
      }
      // ||r~|| <= (1 + 2^-8) ||r|| (bf16 rounding is at most 2^-8 relative per
      // element); 2^-7 also covers the fp32 error of rho.  Stored pre-scaled by
      // the accumulation-error factor D * 2^-22.
      if (half == 0) rn_s[vrow] = (float)D * 0x1p-22f * (rho * (1.0f + 0x1p-7f));
      if (next < a.total_tiles) fetch(next);
      wave_sync();

      // VG: the sign records go to the residual rows' padding
      sketch_signs<D, NRT, VG, P2, SPITCH, VT>(stage, Ssrc, rn_s, a_snmax, rlo, nvalid,
                                   (size_t)bh * a.cap + (size_t)(a.t0 + tbase), a.signs,
                                   stage + 2 * D, lane);
    }
    wave_sync();
    if constexpr (VG) {
      // (the scheduling barriers keep the emission's work from moving into
      // the earlier phases: register pressure)
      __builtin_amdgcn_sched_barrier(0);
      // each lane writes the nibbles of its half of the slot's codes to the
      // slot's stage row (offset made opaque so it is not hoisted out of the
      // tile loop: register pressure); vg_emit_codes regroups the rows
      int off = vrow * P2;
      asm volatile("" : "+v"(off));
      uint8_t *nr = stage + off + (DL / 2) * half;
#pragma unroll
      for (int k = 0; k < DL / 32; ++k)
        *(u32x4 *)(nr + 16 * k) = u32x4{nib[4 * k], nib[4 * k + 1], nib[4 * k + 2], nib[4 * k + 3]};
      wave_sync();
      const size_t slot0 = (size_t)bh * a.cap + (size_t)(a.t0 + tbase);
      vg_emit_codes<BITS, VT, P2, true>(stage, rlo, nvalid, a.codes + slot0 * RECB, lane);
      if constexpr (QJL) vg_emit_signs<VT, P2>(stage + 2 * D, rlo, nvalid, a.signs + slot0 * 16, lane);
      wave_sync();   // the stage takes the next tile
      __builtin_amdgcn_sched_barrier(0);
    }
    if (next < a.total_tiles) stash();
    wave_sync();
  }
}

// Adjacent-pair tree over a stream of block sums b_0, b_1, ... (blk uniform):
// lvl[k] holds a pending left subtree of 2^k blocks.  After the last block of
// a power-of-two count the return value is the root of the same tree that the
// pairwise sum over all leaves builds.
__device__ __forceinline__ float tree_push(float (&lvl)[8], float s, int blk) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (!((blk >> k) & 1)) {
      lvl[k] = s;
      return s;
    }
    s = lvl[k] + s;
  }
  return s;
}

// RB rows of y = Q x: y_i = fma chain over j = 0 .. D-1 ascending from 0.
template <int D, int RB>
__device__ __forceinline__ void dense_rows(cfloat *qb, const float *x, float *yb) {
#pragma unroll
  for (int ii = 0; ii < RB; ++ii) {
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < D; ++j) acc = fmaf(qb[ii * D + j], x[j], acc);
    yb[ii] = acc;
  }
}

// The same RB rows with x split over a lane pair (d = 256): lane l < 32 holds
// x_0 .. x_{D/2-1} of vector l, lane l + 32 the rest.  Each row's chain is
// relayed: the lower lane runs j < D/2 from 0, hands its sum to the upper lane
// (a cross-half shuffle), which continues over j >= D/2, so y_i is the same
// single ascending fma chain.  Both halves work at every step (the lower on
// row ii, the upper on row ii - 1), each reading its own half-row of Q with
// vector loads; y ends in the upper lanes (the lower lanes' yb is scratch).
template <int D, int RB>
__device__ __forceinline__ void dense_rows_relay(const float *Qb, const float (&xh)[D / 2],
                                                 float (&yb)[RB], int half, int lane) {
  constexpr int XN = D / 2;
  float carry = 0.0f;
#pragma unroll
  for (int ii = 0; ii <= RB; ++ii) {
    // idle steps (upper at ii = 0, lower at ii = RB) recompute an in-range row
    const int r = half ? (ii > 0 ? ii - 1 : 0) : (ii < RB ? ii : RB - 1);
    const float *qr = Qb + (size_t)r * D + half * XN;
    float acc = half ? carry : 0.0f;
#pragma unroll
    for (int c = 0; c < XN / 4; ++c) {
      const f32x4v qv = *(const f32x4v *)(qr + 4 * c);
      acc = fmaf(qv[0], xh[4 * c + 0], acc);
      acc = fmaf(qv[1], xh[4 * c + 1], acc);
      acc = fmaf(qv[2], xh[4 * c + 2], acc);
      acc = fmaf(qv[3], xh[4 * c + 3], acc);
    }
    if (ii > 0) yb[ii - 1] = acc;
    carry = __shfl_xor(acc, 32, 64);
  }
}

// ---------------------------------------------------------------------------
// Quantize-on-write with a dense rotation y = Q x (RK_QR; "KVQuant++" thread,
// "Rotation invariance guarantee").  One lane per vector, 64 vectors per wave
// tile, x in registers; Q is read with scalar loads (every lane needs the same
// row at the same time).  At d = 256 (PAIR) a lane pair holds a vector
// (dense_rows_relay), 32 vectors per wave tile, and the upper lane of the pair
// owns everything after y; the sketch is read from memory.  y is formed twice,
// in blocks of 16 rows: first for
// the norm, then for the codes, so only x stays live.  A block's pairwise sum
// of squares is a subtree of the adjacent-pair tree and the block sums are
// combined in that tree's order (tree_push), so nu and rho equal the pairwise
// sums over the whole vector.  Codes of a block are stored as soon as they are
// known; sketch sides stage the bf16 residual rows for sketch_signs.
// ---------------------------------------------------------------------------
template <int D, int BITS, bool QJL, bool BF16, bool VG>
__global__ __launch_bounds__(256) void quantize_dense_kernel(const QuantArgs a) {
  constexpr bool PAIR = D > 128;             // a lane pair per vector
  constexpr int VT = PAIR ? 32 : 64;         // vectors per wave tile
  constexpr int XN = PAIR ? D / 2 : D;       // coordinates of x per lane
  constexpr int RB = D < 16 ? D : 16;        // rows of y per block
  constexpr int NB = D / RB;
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int RECB = D * BITS / 8;
  constexpr int P2 = D * 2 + 16;
  constexpr int SPITCH = PAIR ? D * 2 : P2;
  constexpr int SBYTES = (QJL && !PAIR) ? D * P2 : 16;
  constexpr int RBYTES = QJL ? VT * P2 : 16;
  using LC = LocalCodes<RB, BITS>;
  __shared__ __attribute__((aligned(16))) unsigned char S_s[SBYTES];
  __shared__ __attribute__((aligned(16))) unsigned char res_all[4][RBYTES];
  __shared__ BucketTables<BITS, (D >= 16)> bt;
  __shared__ float rn_all[4][VT];
  static_assert(!VG || D == 128, "token groups exist at d = 128 only");
  __shared__ __attribute__((aligned(16))) uint8_t vrow_all[4][VG ? VT * RECB : 16];
  __shared__ __attribute__((aligned(16))) uint8_t srow_all[4][VG && QJL ? VT * 16 : 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = PAIR ? lane >> 5 : 0;     // PAIR: which half of x this lane holds
  const int vl = PAIR ? lane & 31 : lane;    // this lane's vector in the tile
  const bool own = !PAIR || half == 1;       // the lane that finishes the vector
  const int lead = a.t0 % VT;                // padding rows before t0 in the first tile
  unsigned char *res = res_all[wave];
  float *rn_s = rn_all[wave];
  build_bucket_tables(bt, a.thr, a.cent, tid, 256);
  if constexpr (QJL && !PAIR) stage_sketch<D>(S_s, a.S, tid);
  __syncthreads();
  const unsigned char *Ssrc = PAIR ? (const unsigned char *)a.S : S_s;
  float a_snmax = 0.0f;
  if constexpr (QJL) a_snmax = sketch_row_norm_max<D, SPITCH>(Ssrc, lane);
  cfloat *Qc = (cfloat *)a.Q;

#pragma unroll 1
  for (int tile = blockIdx.x * 4 + wave; tile < a.total_tiles; tile += gridDim.x * 4) {
    const int bh = tile / a.tiles_per_bh;
    const int tt = tile - bh * a.tiles_per_bh;
    const int b = bh / a.H, h = bh - b * a.H;
    const int tbase = tt * VT - lead;
    const int rlo = max(0, -tbase), nvalid = min(VT, a.T - tbase);
    const bool inr = vl >= rlo && vl < nvalid;
    const bool valid = own && inr;           // this lane stores the vector's results
    float x[XN];
#pragma unroll
    for (int i = 0; i < XN; ++i) x[i] = 0.0f;
    if (inr) {
      const unsigned char *src = (const unsigned char *)a.src +
          ((long long)b * a.sb + (long long)h * a.sh + (long long)(tbase + vl) * a.st +
           half * XN) * ESZ;
      if constexpr (BF16) {
#pragma unroll
        for (int c = 0; c < XN / 8; ++c) {
          const u32x4 v = *(const u32x4 *)(src + c * 16);
          x[8 * c + 0] = bf16_lo(v.x); x[8 * c + 1] = bf16_hi(v.x);
          x[8 * c + 2] = bf16_lo(v.y); x[8 * c + 3] = bf16_hi(v.y);
          x[8 * c + 4] = bf16_lo(v.z); x[8 * c + 5] = bf16_hi(v.z);
          x[8 * c + 6] = bf16_lo(v.w); x[8 * c + 7] = bf16_hi(v.w);
        }
      } else {
#pragma unroll
        for (int c = 0; c < XN / 4; ++c) {
          const u32x4 v = *(const u32x4 *)(src + c * 16);
          x[4 * c + 0] = __uint_as_float(v.x); x[4 * c + 1] = __uint_as_float(v.y);
          x[4 * c + 2] = __uint_as_float(v.z); x[4 * c + 3] = __uint_as_float(v.w);
        }
      }
    }
    // pass 1: nu = ||y||
    float lvl[8] = {}, ss = 0.0f;
#pragma unroll 1
    for (int blk = 0; blk < NB; ++blk) {
      float yb[RB];
      if constexpr (PAIR) dense_rows_relay<D, RB>(a.Q + (size_t)blk * RB * D, x, yb, half, lane);
      else dense_rows<D, RB>(Qc + (size_t)blk * RB * D, x, yb);
      ss = tree_push(lvl, pairwise_sumsq<RB>(yb), blk);
    }
    const float nu = sqrtf(ss);
    const float rcp = nu == 0.0f ? 0.0f : 1.0f / nu;
    const size_t slot = (size_t)bh * a.cap + (size_t)(a.t0 + tbase + vl);
    // VG: the record goes to this lane's LDS row, regrouped by vg_emit_codes
    uint8_t *crec = VG ? vrow_all[wave] + lane * RECB : a.codes + slot * RECB;
    // pass 2: codes (and residuals)
    float rl[8] = {}, rs = 0.0f;
#pragma unroll 1
    for (int blk = 0; blk < NB; ++blk) {
      float yb[RB];
      if constexpr (PAIR) dense_rows_relay<D, RB>(a.Q + (size_t)blk * RB * D, x, yb, half, lane);
      else dense_rows<D, RB>(Qc + (size_t)blk * RB * D, x, yb);
      LC lc;
      lc.clear();
#pragma unroll
      for (int ii = 0; ii < RB; ++ii) {
        const float u = yb[ii] * rcp;
        const uint32_t code = bucketize_code<BITS>(u, bt, a.thr);
        lc.put(ii, code);
        if constexpr (QJL) yb[ii] = u - bt.cent[code];
      }
      if (VG || valid) {
        // records are 2-byte aligned (d >= 16): halfword stores; d = 8 records
        // (1 to 4 bytes) are written bytewise
        if constexpr (D < 16) {
          uint32_t img = lc.w[0];
          if constexpr (BITS == 3) img = (lc.w[0] & 0xFFFFu) | (lc.w[LC::NA] << 16);
#pragma unroll
          for (int k = 0; k < RECB; ++k) crec[k] = (uint8_t)(img >> (8 * k));
        } else if constexpr (BITS == 3) {
          uint16_t *p2 = (uint16_t *)(crec + blk * 4);          // 2-bit plane: 4 bytes per block
          p2[0] = (uint16_t)(lc.w[0] & 0xFFFFu);
          p2[1] = (uint16_t)(lc.w[0] >> 16);
          *(uint16_t *)(crec + D / 4 + blk * 2) = (uint16_t)(lc.w[LC::NA] & 0xFFFFu);
        } else {
          uint16_t *pc = (uint16_t *)(crec + blk * (RB * BITS / 8));
#pragma unroll
          for (int k = 0; k < RB * BITS / 16; ++k)
            pc[k] = (uint16_t)((lc.w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu);
        }
      }
      if constexpr (QJL) {
        rs = tree_push(rl, pairwise_sumsq<RB>(yb), blk);
        unsigned char *rrow = res + vl * P2 + blk * RB * 2;
#pragma unroll
        for (int c = 0; c < RB / 8; ++c) {
          if (!own) break;
          uint32_t wv[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const f32x2 pr = {yb[8 * c + 2 * k], yb[8 * c + 2 * k + 1]};
            wv[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
          }
          *(u32x4 *)(rrow + c * 16) = u32x4{wv[0], wv[1], wv[2], wv[3]};
        }
      }
    }
    if (valid) a.norm[slot] = f32_to_f16_bits(nu * a.scale);
    if constexpr (QJL) {
      const float rho = sqrtf(rs);
      if (valid) a.rnorm[slot] = f32_to_f16_bits(rho);
      if (own) rn_s[vl] = (float)D * 0x1p-22f * (rho * (1.0f + 0x1p-7f));
      wave_sync();
      sketch_signs<D, VT / 32, VG, 16, SPITCH>(res, Ssrc, rn_s, a_snmax, rlo, nvalid,
                                               (size_t)bh * a.cap + (size_t)(a.t0 + tbase),
                                               a.signs, srow_all[wave], lane);
      wave_sync();
    }
    if constexpr (VG) {
      wave_sync();
      const size_t slot0 = (size_t)bh * a.cap + (size_t)(a.t0 + tbase);
      vg_emit_codes<BITS, VT>(vrow_all[wave], rlo, nvalid, a.codes + slot0 * RECB, lane);
      if constexpr (QJL) vg_emit_signs<VT>(srow_all[wave], rlo, nvalid, a.signs + slot0 * 16, lane);
      wave_sync();
    }
  }
}

// Read code i of a record (layout as in place_code).
template <int D, int BITS>
__device__ __forceinline__ int get_code(const uint8_t *rec, int i) {
  if constexpr (BITS == 3) {
    const int lo = (rec[(2 * i) >> 3] >> ((2 * i) & 7)) & 3;
    const int hi = (rec[D / 4 + (i >> 3)] >> (i & 7)) & 1;
    return lo | (hi << 2);
  } else {
    return (rec[(i * BITS) >> 3] >> ((i * BITS) & 7)) & ((1 << BITS) - 1);
  }
}

// In-LDS WHT across the D threads of a block (one element per thread).
template <int D>
__device__ __forceinline__ float wht_block(float *t_s, float x) {
  const int i = threadIdx.x;
  t_s[i] = x;
#pragma unroll
  for (int h = 1; h < D; h <<= 1) {
    __syncthreads();
    const float p = t_s[i], q = t_s[i ^ h];
    __syncthreads();
    t_s[i] = (i & h) ? (q - p) : (p + q);
  }
  __syncthreads();
  return t_s[i];
}

// Coordinate i of R^T t for the dense rotation, t in LDS (all D threads).
template <int D>
__device__ __forceinline__ float dense_rotate_back(const float *Q, const float *t_s, int i) {
  float acc = 0.0f;
  // (a bounded unroll: callers forming several coordinates at once would
  // otherwise keep every load of every chain in flight)
#pragma unroll 8
  for (int j = 0; j < D; ++j) acc = fmaf(Q[(size_t)j * D + i], t_s[j], acc);
  return acc;
}

// ---------------------------------------------------------------------------
// Dequantize (parity aid): one block of D threads per record.
//   x^ = ||x|| R^T (C[code] + sqrt(pi/2)/m ||r|| S^T (2 sigma - 1))
// with R^T = H/sqrt(d) (WHT), D H/sqrt(d) (randomized Hadamard), Q^T, or I.
// ---------------------------------------------------------------------------
template <int D, int BITS, int RK, bool QJL>
__global__ __launch_bounds__(D) void dequant_kernel(const DequantArgs a) {
  __shared__ float t_s[D];
  __shared__ float sg_s[D];
  const int v = blockIdx.x, i = threadIdx.x;
  const int bh = v / a.T, t = v - bh * a.T;
  const size_t slot = (size_t)bh * a.cap + (size_t)(a.t0 + t);
  bool vg = false;
  if constexpr (D == 128) vg = a.vg != 0;
  const uint32_t code = vg ? vg_code<BITS>(a.codes, slot, i)
                           : (uint32_t)get_code<D, BITS>(a.codes + slot * (D * BITS / 8), i);
  float val = a.cent[code];
  if constexpr (QJL) {
    const uint8_t *sg = a.signs + slot * (D / 8);
    const uint32_t bit = vg ? vg_sign(a.signs, slot, i) : (uint32_t)((sg[i >> 3] >> (i & 7)) & 1);
    sg_s[i] = bit ? 1.0f : -1.0f;
    __syncthreads();
    float acc = 0.0f;
    for (int k = 0; k < D; ++k) acc = acc + bf16_to_f32(a.S[(size_t)k * D + i]) * sg_s[k];
    val = val + a.coef * f16_bits_to_f32(a.rnorm[slot]) * acc;
  }
  if constexpr (RK == RK_WHT || RK == RK_RHT) val = wht_block<D>(t_s, val) * a.oscale;
  if constexpr (RK == RK_RHT) val = ((a.rsign[i >> 5] >> (i & 31)) & 1u) ? -val : val;
  if constexpr (RK == RK_QR) {
    t_s[i] = val;
    __syncthreads();
    val = dense_rotate_back<D>(a.Q, t_s, i);
  }
  a.out[((size_t)bh * a.T + t) * D + i] = f16_bits_to_f32(a.norm[slot]) * val;
}

// ---------------------------------------------------------------------------
// Query preparation, one block per query row: q' = R q * log2(e)/sqrt(d) with
// the cache's rotation R (q' = H q * log2(e)/d for the WHT, H (D q) for the
// randomized Hadamard, Q q for the dense rotation, q unrotated), and for
// sketched keys S q'.  Rotating q once replaces rotating every key back
// (q . R^T y = (R q) . y); log2(e) lets the scan use exp2.  Output layout
// [b][h_kv][head group][coordinate][GT] puts the GT heads of one coordinate
// side by side, so the scan reads them with scalar loads.
// ---------------------------------------------------------------------------
template <int D, int RK, bool KQ, bool BF16>
__global__ __launch_bounds__(D) void prep_kernel(const PrepArgs a) {
  __shared__ float t_s[D];
  const int row = blockIdx.x, i = threadIdx.x;
  float x = BF16 ? bf16_to_f32(((const uint16_t *)a.q)[(size_t)row * D + i])
                 : ((const float *)a.q)[(size_t)row * D + i];
  if constexpr (RK == RK_RHT) x = ((a.rsign[i >> 5] >> (i & 31)) & 1u) ? -x : x;
  if constexpr (RK == RK_WHT || RK == RK_RHT) x = wht_block<D>(t_s, x);
  if constexpr (RK == RK_QR) {
    t_s[i] = x;
    __syncthreads();
    float acc = 0.0f;
    for (int j = 0; j < D; ++j) acc = fmaf(a.Q[(size_t)i * D + j], t_s[j], acc);
    x = acc;
    __syncthreads();
  }
  x = x * a.qscale;
  size_t dst;
  if (a.nq > 0) {            // multi-query: row = (b * nq + t) * Hq + hq
    const int hq = row % a.Hq, bt = row / a.Hq;
    const int b = bt / a.nq, t = bt - b * a.nq;
    const int hkv = hq / a.G, g = hq - hkv * a.G;
    dst = ((((size_t)b * a.Hkv + hkv) * a.nq + t) * a.G + g) * D + i;
  } else {
    const int b = row / a.Hq, hq = row - b * a.Hq;
    const int hkv = hq / a.G, within = hq - hkv * a.G;
    const int hg = within / a.GT, hh = within - hg * a.GT;
    dst = ((((size_t)b * a.Hkv + hkv) * a.HG + hg) * D + i) * a.GT + hh;
  }
  a.qt[dst] = x;
  if constexpr (KQ) {
    __syncthreads();
    t_s[i] = x;
    __syncthreads();
    float acc = 0.0f;
    for (int k = 0; k < D; ++k) acc = acc + bf16_to_f32(a.S[(size_t)i * D + k]) * t_s[k];
    a.sqt[dst] = acc;
  }
}

// ---------------------------------------------------------------------------
// Decode scan.  One block (4 waves) per (token split, KV head, group of GT
// query heads, batch row); every record of the split is read once and serves
// the GT heads.  Three phases:
//   A  keys, one token per lane: base-2 logit
//        s = n_k * (sum_i q'_i C_K[code_i]  [+ sqrt(pi/2)/m rho_k <S q', 2 sigma - 1>])
//      with q' (and S q') taken from scalar registers; logits stay in LDS.
//   B  the split's exact max M per head, then once per (token, head) the
//      weight w = 2^(s - M), the sum L, and c = w n_v, cq = c rho_v in LDS.
//   C  values: tiles of 64 tokens staged in LDS with coalesced 16-byte loads
//      (next tile prefetched into registers); a token is spread over D/E
//      lanes, each with E coordinates: o' += c C_V[code] (codes looked up two
//      at a time from a pair table) and a += cq (2 sigma - 1).
// The block writes (M, L, o'[D], a[D]) per head; the merge kernel combines the
// splits.
// ---------------------------------------------------------------------------
// One cache record into registers (one lane per token).  Plain loads: the
// record's 16-byte parts are read by separate instructions of the wave, which
// hit the lines the first part brought into L2 (nontemporal loads here
// re-fetched them from memory).
template <int BYTES>
__device__ __forceinline__ void load_rec(const uint8_t *p, uint32_t *w) {
  if constexpr (BYTES % 16 == 0) {
#pragma unroll
    for (int k = 0; k < BYTES / 16; ++k) {
      const u32x4 v = *(const u32x4 *)(p + 16 * k);
      w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
    }
  } else if constexpr (BYTES % 8 == 0) {
#pragma unroll
    for (int k = 0; k < BYTES / 8; ++k) {
      const u32x2 v = *(const u32x2 *)(p + 8 * k);
      w[2 * k] = v.x; w[2 * k + 1] = v.y;
    }
  } else if constexpr (BYTES % 4 == 0) {
#pragma unroll
    for (int k = 0; k < BYTES / 4; ++k) w[k] = *(const uint32_t *)(p + 4 * k);
  } else if constexpr (BYTES == 6) {
    const uint16_t *h = (const uint16_t *)p;
    w[0] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
    w[1] = h[2];
  } else if constexpr (BYTES == 3) {
    w[0] = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16);
  } else if constexpr (BYTES == 1) {
    w[0] = p[0];
  } else {
    static_assert(BYTES == 2, "record size");
    w[0] = *(const uint16_t *)p;
  }
}

// Codes of one lane's E-coordinate slice g of a record in LDS: w0 holds the
// low (or only) bits, w1 the 1-bit plane of 3-bit codes or the upper half of
// 4-bit codes when E = 16.
template <int D, int BITS, int E>
__device__ __forceinline__ void lds_codes(const uint8_t *r, int g, uint32_t &w0, uint32_t &w1) {
  if constexpr (E == 16) {
    if constexpr (BITS == 4) {
      const u32x2 v = *(const u32x2 *)(r + g * 8);
      w0 = v.x;
      w1 = v.y;
    } else if constexpr (BITS == 3) {
      w0 = (uint32_t) * (const uint16_t *)(r + g * 4) | ((uint32_t) * (const uint16_t *)(r + g * 4 + 2) << 16);
      w1 = *(const uint16_t *)(r + D / 4 + g * 2);
    } else if constexpr (BITS == 2) {
      w0 = *(const uint32_t *)(r + g * 4);
      w1 = 0u;
    } else {
      w0 = *(const uint16_t *)(r + g * 2);
      w1 = 0u;
    }
  } else {
    if constexpr (BITS == 4) {
      w0 = *(const uint32_t *)(r + g * 4);
      w1 = 0u;
    } else if constexpr (BITS == 3 && D == 8) {
      // 3-byte records: rows at odd addresses, so byte reads
      w0 = (uint32_t)r[0] | ((uint32_t)r[1] << 8);
      w1 = r[2];
    } else if constexpr (BITS == 3) {
      w0 = *(const uint16_t *)(r + g * 2);
      w1 = r[D / 4 + g];
    } else if constexpr (BITS == 2) {
      w0 = *(const uint16_t *)(r + g * 2);
      w1 = 0u;
    } else {
      w0 = r[g];
      w1 = 0u;
    }
  }
}

// The first nb bytes (below 16) of a 16-byte piece, zero-extended: the last
// piece of a split's value segment may end inside the piece (records of 1, 2,
// 3, 6, 8, 12 or 24 bytes), and the bytes after it may lie past the end of
// the caller's buffer.  Halfword reads for even nb (the records of 2-byte
// multiples start 2-byte aligned), byte reads otherwise.
__device__ __forceinline__ u32x4 load_piece_tail(const uint8_t *p, int nb) {
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if ((nb & 1) == 0 && (((uintptr_t)p) & 1) == 0) {
    for (int i = 0; i < nb; i += 2) w[i >> 2] |= (uint32_t)(*(const uint16_t *)(p + i)) << (8 * (i & 2));
  } else {
    for (int i = 0; i < nb; ++i) w[i >> 2] |= (uint32_t)p[i] << (8 * (i & 3));
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// Pair-table index of coordinates (2p, 2p+1) of a whole record held as words
// (same index convention as pair_index).
template <int D, int BITS>
__device__ __forceinline__ uint32_t rec_pair(const uint32_t *w, int p) {
  if constexpr (BITS == 4) return (w[p >> 2] >> (8 * (p & 3))) & 255u;
  if constexpr (BITS == 3)   // the 1-bit plane starts at bit 2 D (byte D / 4)
    return ((w[p >> 3] >> (4 * (p & 7))) & 15u) |
           (((w[(2 * D + 2 * p) >> 5] >> ((2 * D + 2 * p) & 31)) & 3u) << 4);
  if constexpr (BITS == 2) return (w[p >> 3] >> (4 * (p & 7))) & 15u;
  return (w[p >> 4] >> (2 * (p & 15))) & 3u;
}

// Codes of coordinate pair p of a lane's E-coordinate slice (words from
// lds_codes), as an index into the pair table.  Widths 1, 2, 4: the two codes'
// bits are adjacent (index = code_a | code_b << BITS).  Width 3: the pair's
// nibble of the 2-bit plane, then its two bits of the 1-bit plane.
template <int BITS>
__device__ __forceinline__ uint32_t pair_index(uint32_t w0, uint32_t w1, int p) {
  if constexpr (BITS == 4) return ((p < 4 ? w0 : w1) >> (8 * (p & 3))) & 255u;
  if constexpr (BITS == 3) return ((w0 >> (4 * p)) & 15u) | (((w1 >> (2 * p)) & 3u) << 4);
  if constexpr (BITS == 2) return (w0 >> (4 * p)) & 15u;
  return (w0 >> (2 * p)) & 3u;
}
// The two codes a pair-table index stands for.
template <int BITS>
__device__ __forceinline__ void pair_codes(int idx, int &ca, int &cb) {
  if constexpr (BITS == 3) {
    ca = (idx & 3) | (((idx >> 4) & 1) << 2);
    cb = ((idx >> 2) & 3) | (((idx >> 5) & 1) << 2);
  } else {
    ca = idx & ((1 << BITS) - 1);
    cb = idx >> BITS;
  }
}

// Sum over each aligned group of N lanes (N = 1, 2, 4, 8, 16), result in every
// lane of the group, with DPP lane permutes (no LDS traffic): quad_perm swaps
// lanes 1 and 2 apart, row_half_mirror pairs the two quads of 8 lanes,
// row_mirror pairs the two halves of a 16-lane row.  Partners add the same two
// operands, so every lane of a group ends with the same bits.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  if constexpr (N >= 4)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  if constexpr (N >= 8)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  if constexpr (N >= 16)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

// 2^x with the hardware instruction (results below 2^-126 flush to zero, which
// only drops softmax weights that are negligible anyway).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// A uniform zero the compiler cannot see through: added to the scalar-load
// offsets inside the token loop, it keeps the query loads in the loop (one
// chunk of SGPRs live at a time) instead of hoisting all of them.
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("s_mov_b32 %0, 0" : "=s"(z));
  return z;
}


// An empty asm the value passes through: the compiler cannot fold the masks
// that built it into each later byte extract (which would cost two
// instructions per extract instead of one).
__device__ __forceinline__ void pin_reg(uint32_t &x) { asm("" : "+v"(x)); }

// Byte layout of one value tile of TT tokens in LDS: value codes, then value
// sign bits (sketched values).
template <int D, int VB, bool VQ, int TT>
struct VTile {
  static constexpr int VREC = D * VB / 8, SREC = D / 8;
  static constexpr int VC = 0;
  static constexpr int VS = VC + TT * VREC;
  static constexpr int BYTES = VS + (VQ ? TT * SREC : 0);
  static constexpr int NCH = BYTES / 16;
  static_assert(BYTES % 16 == 0 && VS % 16 == 0, "tile segments must be 16-byte multiples");
};

// Split merge of one query row (b, hq), one block of 256 threads: the
// log-sum-exp weights of the splits, the weighted sums of their partials,
// o' + sqrt(pi/2)/m S^T a (sketched values), the inverse rotation and the
// division by L (and the full-precision window, if any).  Every load that does
// not depend on another (the split maxima, the partial columns, the columns
// of S, the window partial) is issued at the start, so the row costs about one
// memory latency; the split weights stay in registers (lane s of the wave
// holds split s of the current 64) and the Walsh-Hadamard transform runs
// across the lanes of one wave.
template <int D, bool VQ>
__global__ __launch_bounds__(256) void merge_kernel(const DecodeArgs a) {
  constexpr int NS = 2 + 2 * D, NC = NS - 1;         // partial floats, columns merged
  constexpr int NIT = (NC + 255) / 256;              // columns per thread
  constexpr int U = 16;                              // splits per load batch
  // S^T a: KS threads per coordinate, KL rows of S each (in registers when
  // few, else read in the loop)
  constexpr int KS = (256 / D) < D ? (256 / D) : D, KL = D / KS;
  constexpr bool SREG = KL <= 64;
  __shared__ __attribute__((aligned(16))) float res[NS];    // merged L, o', a (by column)
  __shared__ __attribute__((aligned(16))) float sta[256];   // S^T a partial sums
  __shared__ __attribute__((aligned(16))) float wv[D];
  const int tid = threadIdx.x, lane = tid & 63;
  const int row = blockIdx.x;                        // b * Hq + hq
  const int splits = a.splits;
  const float *pb = a.part + (size_t)row * splits * NS;

  // columns of S for this thread's share of S^T a: every thread at d >= 16
  // (KS d = 256); at d = 8 threads tid >= KS d read a valid row and drop it
  // (no per-load branch: the loads stay in flight together)
  const int si = tid % D;
  const bool sthr = KS * D >= 256 || tid < KS * D;
  const int sk0 = sthr ? (tid / D) * KL : 0;
  uint16_t sv[VQ && SREG ? KL : 1];
  if constexpr (VQ && SREG) {
#pragma unroll
    for (int k = 0; k < KL; ++k) sv[k] = ((const uint16_t *)a.S)[(size_t)(sk0 + k) * D + si];
  }
  // the window partial of this thread's output coordinate
  float wm = -INFINITY, wl = 0.0f, wo = 0.0f;
  if (a.wpart && tid < D) {
    const float *wp = a.wpart + (size_t)row * (2 + D);
    wm = wp[0];
    wl = wp[1];
    wo = wp[2 + tid];
  }
  auto load_batch = [&](int s0, float (&v)[NIT][U]) {
#pragma unroll
    for (int j = 0; j < NIT; ++j) {
      const int item = tid + 256 * j;
      const bool ok = item < NC;
      const float *src = pb + (size_t)s0 * NS + 1 + (ok ? item : 0);
#pragma unroll
      for (int u = 0; u < U; ++u) v[j][u] = (ok && s0 + u < splits) ? src[(size_t)u * NS] : 0.0f;
    }
  };
  float v[NIT][U];
  load_batch(0, v);
  // maximum over the splits (every wave computes it: no barrier)
  const float ms0 = lane < splits ? pb[(size_t)lane * NS] : -INFINITY;
  float m = ms0;
  for (int s = lane + 64; s < splits; s += 64) m = fmaxf(m, pb[(size_t)s * NS]);
  m = wave_max(m);

  float acc[NIT];
#pragma unroll
  for (int j = 0; j < NIT; ++j) acc[j] = 0.0f;
  float w = 0.0f;
  for (int s0 = 0; s0 < splits; s0 += U) {
    if ((s0 & 63) == 0) {
      const int sl = s0 + lane;
      const float ms = s0 == 0 ? ms0 : (sl < splits ? pb[(size_t)sl * NS] : -INFINITY);
      w = (ms == -INFINITY) ? 0.0f : fast_exp2(ms - m);
    }
    float vn[NIT][U];
    if (s0 + U < splits) {
      load_batch(s0 + U, vn);
    } else {
#pragma unroll
      for (int j = 0; j < NIT; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u) vn[j][u] = 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wu = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), (s0 & 63) + u));
#pragma unroll
      for (int j = 0; j < NIT; ++j) acc[j] = fmaf(wu, v[j][u], acc[j]);
    }
#pragma unroll
    for (int j = 0; j < NIT; ++j)
#pragma unroll
      for (int u = 0; u < U; ++u) v[j][u] = vn[j][u];
  }
#pragma unroll
  for (int j = 0; j < NIT; ++j)
    if (tid + 256 * j < NC) res[1 + tid + 256 * j] = acc[j];
  __syncthreads();

  // o' (+ sqrt(pi/2)/m S^T a): KS partial sums per coordinate, added in order
  if constexpr (VQ) {
    float t = 0.0f;
    if constexpr (SREG) {
#pragma unroll
      for (int k = 0; k < KL; ++k) t = fmaf(bf16_to_f32(sv[k]), res[2 + D + sk0 + k], t);
    } else {
#pragma unroll 8
      for (int k = 0; k < KL; ++k)
        t = fmaf(bf16_to_f32(((const uint16_t *)a.S)[(size_t)(sk0 + k) * D + si]),
                 res[2 + D + sk0 + k], t);
    }
    sta[tid] = sthr ? t : 0.0f;
    __syncthreads();
  }
  if (tid < 64) {
    // lane l holds coordinates l + 64 e, e < PL
    constexpr int PL = D > 64 ? D / 64 : 1;
    float x[PL];
#pragma unroll
    for (int e = 0; e < PL; ++e) {
      const int i = lane + 64 * e;
      float val = 0.0f;
      if (i < D) {
        val = res[2 + i];
        if constexpr (VQ) {
          float u = 0.0f;
#pragma unroll
          for (int p = 0; p < KS; ++p) u += sta[p * D + i];
          val = fmaf(a.vcoef, u, val);
        }
      }
      x[e] = val;
    }
    if (a.rk == RK_WHT || a.rk == RK_RHT) {
      // pairs (i, i + h): the lane with bit h clear keeps the sum, the other
      // the difference (lower minus upper)
#pragma unroll
      for (int h = 1; h < (D < 64 ? D : 64); h <<= 1) {
#pragma unroll
        for (int e = 0; e < PL; ++e) {
          const float y = __shfl_xor(x[e], h, 64);
          x[e] = (lane & h) ? (y - x[e]) : (x[e] + y);
        }
      }
      // stages h = 64 e' within the lane: pairs (e, e + e')
#pragma unroll
      for (int hs = 1; hs < PL; hs <<= 1) {
#pragma unroll
        for (int e = 0; e < PL; ++e) {
          if (e & hs) continue;
          const float lo = x[e], hi = x[e + hs];
          x[e] = lo + hi;
          x[e + hs] = lo - hi;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < PL; ++e)
      if (lane + 64 * e < D) wv[lane + 64 * e] = x[e];
  }
  __syncthreads();
  if (tid < D) {
    const int i = tid;
    float num = wv[i] * a.oscale, den = res[1];
    if (a.rk == RK_RHT && ((a.rsign[i >> 5] >> (i & 31)) & 1u)) num = -num;
    if (a.rk == RK_QR) num = dense_rotate_back<D>(a.Q, wv, i);
    if (a.wpart) {
      // one more log-sum-exp merge, in the original space (the window partial
      // is already there)
      const float mc = m, mu = wm;
      const float mm = fmaxf(mc, mu);
      const float ac = (mc == -INFINITY) ? 0.0f : fast_exp2(mc - mm);
      const float au = (mu == -INFINITY) ? 0.0f : fast_exp2(mu - mm);
      num = ac * num + au * wo;
      den = ac * den + au * wl;
    }
    a.out[(size_t)row * D + i] = num / den;
  }
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));


template <int D, int KB, bool KQ, int VB, bool VQ, int GT>
// (three blocks per CU: registers <= 168)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void decode_kernel(
    const DecodeArgs a) {
  constexpr int E = (GT >= 4 || D < 16) ? 8 : 16;   // value coordinates per lane
  constexpr int L = D / E;                           // lanes sharing a token group in phase C
  constexpr int GPW = 64 / L;                        // token groups per wave
  constexpr int TG = 4;                              // tokens per group
  constexpr int TT = (1024 / L) < 256 ? (1024 / L) : 256;  // tokens per value tile
  constexpr int NWA = TT / (GPW * TG);               // waves that own groups of a tile
  constexpr int NGT = TT / TG;                       // groups per tile
  constexpr int NS = 2 + 2 * D;
  constexpr int TPS_MAX = kScanWbufFloats / (2 * GT);
  constexpr int KBYTES = D * KB / 8, KW = (KBYTES + 3) / 4;
  constexpr int SBYTES = D / 8, SW = (SBYTES + 3) / 4;
  constexpr int NPAIR = 1 << (2 * VB);
  constexpr int KPAIR = 1 << (2 * KB);
  using TL = VTile<D, VB, VQ, TT>;
  constexpr int NPT = (TL::NCH + 255) / 256;         // 16-B chunks per thread per tile
  constexpr int TSH = GT == 4 ? 4 : (GT == 2 ? 3 : 2);  // log2 of a table entry's bytes
  constexpr int EPI = GT * NS;                       // epilogue floats (reuses wbuf)
  static_assert(TPS_MAX % TT == 0, "split budget must be whole tiles");
  static_assert(NWA >= 1 && NWA <= 4 && E % 8 == 0, "phase C mapping");
  static_assert(EPI <= kScanWbufFloats, "epilogue staging must fit the logit buffer");
  static_assert(GT * (256 + NS) <= kScanWbufFloats, "merge staging must fit the logit buffer");

  __shared__ __attribute__((aligned(16))) float wbuf[kScanWbufFloats];
  __shared__ __attribute__((aligned(16))) uint8_t tile[TL::BYTES];
  // sign tables of the tile's token groups: for group g and 4-bit mask m,
  // sum_i (2 m_i - 1) cq[4g + i] per head
  __shared__ __attribute__((aligned(16))) float tbl[VQ ? NGT * 16 * GT : 1];
  __shared__ __attribute__((aligned(8))) f32x2 kp_s[KPAIR];
  __shared__ __attribute__((aligned(8))) f32x2 vp_s[NPAIR];
  __shared__ float red_s[4][GT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x;
  const int hkv = blockIdx.y / a.HG, hg = blockIdx.y - (blockIdx.y / a.HG) * a.HG;
  const int b = blockIdx.z;
  const int hq0 = hkv * a.Gtot + hg * GT;
  const size_t unit = (size_t)b * a.Hkv + hkv;
  const size_t unitg = unit * a.HG + hg;
  for (int p = tid; p < KPAIR; p += 256) {
    int ca, cb;
    pair_codes<KB>(p, ca, cb);
    kp_s[p] = f32x2{a.kcent[ca], a.kcent[cb]};
  }
  for (int p = tid; p < NPAIR; p += 256) {
    int ca, cb;
    pair_codes<VB>(p, ca, cb);
    vp_s[p] = f32x2{a.vcent[ca], a.vcent[cb]};
  }

  // logits, then weights c = w n_v per (token, head) in plane wc; cq = c rho_v
  // in plane wq (16 bytes per token at four heads: linear b128 accesses)
  float *const wc = wbuf;
  float *const wq = wbuf + TPS_MAX * GT;
  const int t_lo = split * a.tps;
  const int t_hi = min(a.n_ctx, t_lo + a.tps);
  const int nloc = t_hi > t_lo ? t_hi - t_lo : 0;
  const size_t rec0 = unit * a.cap + a.t0 + t_lo;    // first record of the split
  __syncthreads();

  // value tiles: thread tid copies 16-byte chunks tid + 256k of each tile;
  // PD tiles are in flight in registers (the first ones requested before
  // phase A, so they arrive while the keys are scored)
  constexpr int PD = 2;
  const int nround = (nloc + TT - 1) / TT * TT;
  const int ntiles = nround / TT;
  const uint8_t *cbase[NPT];
  int crec[NPT], coff[NPT];
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const int byte = (tid + 256 * k) * 16;
    const uint8_t *base = nullptr;
    int rec = 1, start = 0;
    if (byte < TL::VS) { base = a.vc; rec = TL::VREC; start = TL::VC; }
    else if (byte < TL::BYTES) { base = a.vs; rec = TL::SREC; start = TL::VS; }
    cbase[k] = base ? base + rec0 * rec : nullptr;
    crec[k] = rec;
    coff[k] = byte - start;
  }
  u32x4 pf[PD][NPT];
  auto fetch = [&](int it, u32x4 *dst) {
    const int nv = min(TT, nloc - it * TT);
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      dst[k] = u32x4{0u, 0u, 0u, 0u};
      if (it < ntiles && cbase[k]) {
        const uint8_t *src = cbase[k] + (size_t)it * TT * crec[k] + coff[k];
        const int end = nv * crec[k];
        if constexpr (TL::VREC % 16 == 0 && TL::SREC % 16 == 0) {
          // whole records per piece: a piece is either valid or past the end
          if (coff[k] < end) dst[k] = __builtin_nontemporal_load((const u32x4 *)src);
        } else {
          if (coff[k] + 16 <= end) dst[k] = __builtin_nontemporal_load((const u32x4 *)src);
          else if (coff[k] < end) dst[k] = load_piece_tail(src, end - coff[k]);
        }
      }
    }
  };
  auto stash = [&](const u32x4 *src) {
#pragma unroll
    for (int k = 0; k < NPT; ++k)
      if (cbase[k]) *(u32x4 *)(tile + (tid + 256 * k) * 16) = src[k];
  };
#pragma unroll
  for (int j = 0; j < PD; ++j) fetch(j, pf[j]);

  // ---- phase A: logits, one token per lane -------------------------------
  cfloat *qc = (cfloat *)(a.qt + unitg * D * GT);
  cfloat *sc = (cfloat *)(a.sqt + unitg * D * GT);
  const uint8_t *kc_p = a.kc + rec0 * KBYTES;
  const uint8_t *ks_p = KQ ? a.ks + rec0 * SBYTES : nullptr;
  const uint16_t *kn_p = a.kn + rec0;
  const uint16_t *kr_p = KQ ? a.kr + rec0 : nullptr;
  const uint16_t *vn_p = a.vn + rec0;
  const uint16_t *vr_p = VQ ? a.vr + rec0 : nullptr;
  float mx[GT];
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) mx[hh] = -INFINITY;

  uint32_t kw[KW], ksw[SW];
  float nk = 0.0f, rk = 0.0f;
  uint32_t vnr = 0u;   // fp16 bits of the value norm (low) and residual norm (high)
  auto kload = [&](int tl, uint32_t *w, uint32_t *sw, float &n, float &r, uint32_t &vv) {
    if (tl < nloc) {
      load_rec<KBYTES>(kc_p + (size_t)tl * KBYTES, w);
      n = f16_bits_to_f32(__builtin_nontemporal_load(kn_p + tl));
      vv = (uint32_t)__builtin_nontemporal_load(vn_p + tl) |
           (VQ ? (uint32_t)__builtin_nontemporal_load(vr_p + tl) << 16 : 0u);
      if constexpr (KQ) {
        load_rec<SBYTES>(ks_p + (size_t)tl * SBYTES, sw);
        r = f16_bits_to_f32(__builtin_nontemporal_load(kr_p + tl));
      }
    } else {
#pragma unroll
      for (int k = 0; k < KW; ++k) w[k] = 0u;
#pragma unroll
      for (int k = 0; k < SW; ++k) sw[k] = 0u;
      n = 0.0f;
      r = 0.0f;
      vv = 0u;
    }
  };
  kload(wave * 64 + lane, kw, ksw, nk, rk, vnr);
  for (int base = wave * 64; base < nloc; base += 256) {
    uint32_t nw[KW], nsw[SW];
    float nnk, nrk;
    uint32_t nvnr;
    kload(base + 256 + lane, nw, nsw, nnk, nrk, nvnr);    // prefetch the next round
    const int z = opaque_zero();
    float acc[GT], sk[GT];
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      acc[hh] = 0.0f;
      sk[hh] = 0.0f;
    }
#pragma unroll
    for (int p = 0; p < D / 2; ++p) {
      const f32x2 ck = kp_s[rec_pair<D, KB>(kw, p)];
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) {
        acc[hh] = fmaf(qc[z + (2 * p) * GT + hh], ck.x, acc[hh]);
        acc[hh] = fmaf(qc[z + (2 * p + 1) * GT + hh], ck.y, acc[hh]);
      }
    }
    if constexpr (KQ) {
#pragma unroll
      for (int i = 0; i < D; ++i) {
        const float sg = ((ksw[i >> 5] >> (i & 31)) & 1u) ? 1.0f : -1.0f;
#pragma unroll
        for (int hh = 0; hh < GT; ++hh) sk[hh] = fmaf(sc[z + i * GT + hh], sg, sk[hh]);
      }
    }
    const int tl = base + lane;
    if (tl < nloc) {
      float s[GT];
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) {
        if constexpr (KQ) s[hh] = nk * fmaf(a.kcoef * rk, sk[hh], acc[hh]);
        else s[hh] = nk * acc[hh];
        mx[hh] = fmaxf(mx[hh], s[hh]);
      }
      float *dst = wc + tl * GT;
      if constexpr (GT == 4) *(float4 *)dst = float4{s[0], s[1], s[2], s[3]};
      else if constexpr (GT == 2) *(f32x2 *)dst = f32x2{s[0], s[1]};
      else dst[0] = s[0];
      *(uint32_t *)(wq + tl * GT) = vnr;
    }
#pragma unroll
    for (int k = 0; k < KW; ++k) kw[k] = nw[k];
#pragma unroll
    for (int k = 0; k < SW; ++k) ksw[k] = nsw[k];
    nk = nnk;
    rk = nrk;
    vnr = nvnr;
  }
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    const float m = wave_max(mx[hh]);
    if (lane == 0) red_s[wave][hh] = m;
  }
  __syncthreads();

  // ---- phase B: exact split max, weights once per (token, head) ----------
  float M[GT], Lp[GT];
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    M[hh] = fmaxf(fmaxf(red_s[0][hh], red_s[1][hh]), fmaxf(red_s[2][hh], red_s[3][hh]));
    Lp[hh] = 0.0f;
  }
  for (int tl = tid; tl < nround; tl += 256) {
    float c[GT], cq[GT];
    if (tl < nloc) {
      const uint32_t nvr = *(const uint32_t *)(wq + tl * GT);   // stored in phase A
      const float nv = f16_bits_to_f32((uint16_t)(nvr & 0xFFFFu));
      const float rv = VQ ? f16_bits_to_f32((uint16_t)(nvr >> 16)) : 0.0f;
      const float *src = wc + tl * GT;
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) {
        const float w = fast_exp2(src[hh] - M[hh]);
        Lp[hh] += w;
        c[hh] = w * nv;
        cq[hh] = c[hh] * rv;
      }
    } else {
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) {
        c[hh] = 0.0f;
        cq[hh] = 0.0f;
      }
    }
    float *dc = wc + tl * GT, *dq = wq + tl * GT;
    if constexpr (GT == 4) {
      *(float4 *)dc = float4{c[0], c[1], c[2], c[3]};
      *(float4 *)dq = float4{cq[0], cq[1], cq[2], cq[3]};
    } else if constexpr (GT == 2) {
      *(f32x2 *)dc = f32x2{c[0], c[1]};
      *(f32x2 *)dq = f32x2{cq[0], cq[1]};
    } else {
      dc[0] = c[0];
      dq[0] = cq[0];
    }
  }

  // ---- phase C: values ---------------------------------------------------
  // Lane (gs, lg) owns coordinates [lg*E, lg*E + E) of token group
  // wave*GPW + gs of every tile (4 consecutive tokens).  Sign bits of the 4
  // tokens are transposed so that each coordinate's 4 bits form a table index.
  const int lg = lane % L, gs = lane / L;
  const int grp = wave * GPW + gs;
  const bool active = wave < NWA;
  float o[GT][E], av[GT][E];
#pragma unroll
  for (int hh = 0; hh < GT; ++hh)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      o[hh][e] = 0.0f;
      av[hh][e] = 0.0f;
    }
  // tables of tile `it` from the weights cq (zero past the split's end)
  auto build_tables = [&](int it) {
    if constexpr (VQ) {
      for (int idx = tid; idx < NGT * 16; idx += 256) {
        const int g = idx >> 4, m = idx & 15;
        const float *cqp = wq + (it * TT + g * TG) * GT;
        float acc[GT];
#pragma unroll
        for (int hh = 0; hh < GT; ++hh) acc[hh] = 0.0f;
#pragma unroll
        for (int i = 0; i < TG; ++i) {
          const float sg = ((m >> i) & 1) ? 1.0f : -1.0f;
#pragma unroll
          for (int hh = 0; hh < GT; ++hh) acc[hh] = fmaf(sg, cqp[i * GT + hh], acc[hh]);
        }
        float *dst = tbl + idx * GT;
        if constexpr (GT == 4) *(float4 *)dst = float4{acc[0], acc[1], acc[2], acc[3]};
        else if constexpr (GT == 2) *(f32x2 *)dst = f32x2{acc[0], acc[1]};
        else dst[0] = acc[0];
      }
    }
  };
  // add the table entries of 8 coordinates whose 4-token sign bits are in w
  // (byte i = token i, bit e = coordinate e0 + e)
  auto sign_terms = [&](uint32_t w, int e0) {
    // 4x8 bit transpose by four delta swaps: afterwards nibble e holds the
    // bits of coordinate e for tokens 0..3
    auto dswap = [](uint32_t x, int sh, uint32_t m) {
      const uint32_t t = ((x >> sh) ^ x) & m;
      return x ^ t ^ (t << sh);
    };
    uint32_t y = dswap(w, 7, 0x00AA00AAu);
    y = dswap(y, 14, 0x0000CCCCu);
    y = dswap(y, 4, 0x00F000F0u);
    y = dswap(y, 8, 0x0000FF00u);
    uint32_t lo = (y << TSH) & (0x0F0F0F0Fu << TSH);          // even coordinates
    uint32_t hi = (y >> (4 - TSH)) & (0x0F0F0F0Fu << TSH);    // odd coordinates
    pin_reg(lo);
    pin_reg(hi);
    const uint8_t *tg = (const uint8_t *)tbl + (size_t)grp * 16 * GT * 4;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t off = (((e & 1) ? hi : lo) >> (8 * (e >> 1))) & 0xFFu;
      const float *t = (const float *)(tg + off);
      if constexpr (GT == 4) {
        const float4 v = *(const float4 *)t;
        av[0][e0 + e] += v.x;
        av[1][e0 + e] += v.y;
        av[2][e0 + e] += v.z;
        av[3][e0 + e] += v.w;
      } else if constexpr (GT == 2) {
        const f32x2 v = *(const f32x2 *)t;
        av[0][e0 + e] += v.x;
        av[1][e0 + e] += v.y;
      } else {
        av[0][e0 + e] += t[0];
      }
    }
  };
  __syncthreads();   // weights of phase B are in LDS
  if constexpr (VQ) {
    if (ntiles > 0) build_tables(0);
  }
  for (int it0 = 0; it0 < ntiles; it0 += PD) {
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      const int it = it0 + j;
      if (it >= ntiles) break;
      // tile `it` is in pf[j]; refill pf[j] with tile it + PD
      stash(pf[j]);
      fetch(it + PD, pf[j]);
      __syncthreads();   // tile `it` (and its sign tables) are in LDS
      if (active) {
        const int tr0 = grp * TG;
        float c[TG][GT];
#pragma unroll
        for (int i = 0; i < TG; ++i) {
          const float *wsrc = wc + (it * TT + tr0 + i) * GT;
#pragma unroll
          for (int hh = 0; hh < GT; ++hh) c[i][hh] = wsrc[hh];
        }
#pragma unroll
        for (int i = 0; i < TG; ++i) {
          uint32_t vw0, vw1;
          lds_codes<D, VB, E>(tile + TL::VC + (tr0 + i) * TL::VREC, lg, vw0, vw1);
#pragma unroll
          for (int p = 0; p < E / 2; ++p) {
            const f32x2 cv = vp_s[pair_index<VB>(vw0, vw1, p)];
#pragma unroll
            for (int hh = 0; hh < GT; ++hh) {
              o[hh][2 * p] = fmaf(c[i][hh], cv.x, o[hh][2 * p]);
              o[hh][2 * p + 1] = fmaf(c[i][hh], cv.y, o[hh][2 * p + 1]);
            }
          }
        }
        if constexpr (VQ) {
          const uint8_t *sb = tile + TL::VS + tr0 * TL::SREC;
          if constexpr (E == 8) {
            uint32_t w = 0u;
#pragma unroll
            for (int i = 0; i < TG; ++i) w |= (uint32_t)sb[i * TL::SREC + lg] << (8 * i);
            sign_terms(w, 0);
          } else {
            uint32_t h[TG];
#pragma unroll
            for (int i = 0; i < TG; ++i) h[i] = *(const uint16_t *)(sb + i * TL::SREC + lg * 2);
            const uint32_t x01 = h[0] | (h[1] << 16), x23 = h[2] | (h[3] << 16);
            sign_terms(__builtin_amdgcn_perm(x23, x01, 0x06040200u), 0);
            sign_terms(__builtin_amdgcn_perm(x23, x01, 0x07050301u), 8);
          }
        }
      }
      __syncthreads();
      if constexpr (VQ) {
        if (it + 1 < ntiles) build_tables(it + 1);
      }
    }
  }

  // ---- epilogue: sum token slots (lanes), then waves; L over threads -------
#pragma unroll
  for (int off = L; off < 64; off <<= 1) {
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        o[hh][e] += __shfl_xor(o[hh][e], off, 64);
        if constexpr (VQ) av[hh][e] += __shfl_xor(av[hh][e], off, 64);
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    float l = Lp[hh];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) l += __shfl_xor(l, off, 64);
    Lp[hh] = l;
  }
  // waves fold their partial sums into one [GT][NS] buffer in turn (the logit
  // buffer is dead now); lane 0 of each wave adds its L
  float *wst = wbuf;
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
      if (gs == 0) {
#pragma unroll
        for (int hh = 0; hh < GT; ++hh) {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            float *po = wst + hh * NS + 2 + lg * E + e;
            float *pa = wst + hh * NS + 2 + D + lg * E + e;
            const float ov = o[hh][e], avv = VQ ? av[hh][e] : 0.0f;
            *po = (w == 0) ? ov : *po + ov;
            *pa = (w == 0) ? avv : *pa + avv;
          }
        }
      }
      if (lane == 0) {
#pragma unroll
        for (int hh = 0; hh < GT; ++hh) wst[hh * NS + 1] = (w == 0) ? Lp[hh] : wst[hh * NS + 1] + Lp[hh];
      }
    }
    __syncthreads();
  }
  // the merge kernel that follows on the stream combines the splits
  for (int idx = tid; idx < GT * NS; idx += 256) {
    const int hh = idx / NS, k = idx - hh * NS;
    float *dst = a.part + (((size_t)b * a.Hq + hq0 + hh) * a.splits + split) * NS;
    dst[k] = (k == 0) ? (nloc > 0 ? M[hh] : -INFINITY) : wst[idx];
  }
}

// ---------------------------------------------------------------------------
// Full-precision window ("Your KV cache is not a bit problem but a geometry
// problem": keep the most recent tokens, and attention-sink tokens, at full
// precision next to the quantized cache).  One block per query row computes
// the exact partial over the window tokens: base-2 logits s_j = log2(e)
// q.k_j / sqrt(d), their max M, L = sum 2^(s_j - M) and o = sum 2^(s_j - M) v_j,
// which the scan's merge combines with the compressed splits.
// ---------------------------------------------------------------------------
template <int D, bool QB, bool WB>
__global__ __launch_bounds__(256) void window_kernel(const WindowArgs a) {
  __shared__ float qf[D];
  __shared__ float sj[KVQ_WINDOW_MAX];
  __shared__ float red[4];
  __shared__ float po[2][D];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = row / (a.Hq * a.nq), hq = row % a.Hq;
  const int hkv = hq / (a.Hq / a.Hkv);
  const size_t base = ((size_t)b * a.Hkv + hkv) * a.n_win * D;
  for (int i = tid; i < D; i += 256) {
    const float x = QB ? bf16_to_f32(((const uint16_t *)a.q)[(size_t)row * D + i])
                       : ((const float *)a.q)[(size_t)row * D + i];
    qf[i] = x * a.qscale;
  }
  __syncthreads();
  auto wval = [&](const void *p, size_t idx) {
    return WB ? bf16_to_f32(((const uint16_t *)p)[idx]) : ((const float *)p)[idx];
  };
  // scores and weighted sums accumulate in fp64 (a window is at most
  // KVQ_WINDOW_MAX tokens; fp32 chains of d = 256 terms would cost most of the
  // output's 1e-5 relative budget)
  float m = -INFINITY;
  for (int j = tid; j < a.n_win; j += 256) {
    double s = 0.0;
    for (int i = 0; i < D; ++i) s = fma((double)qf[i], (double)wval(a.wk, base + (size_t)j * D + i), s);
    sj[j] = (float)s;
    m = fmaxf(m, sj[j]);
  }
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float l = 0.0f;
  for (int j = tid; j < a.n_win; j += 256) {
    const float w = fast_exp2(sj[j] - M);
    sj[j] = w;
    l += w;
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) l += __shfl_xor(l, off, 64);
  if (lane == 0) red[wave] = l;
  __syncthreads();
  // o: two token halves per coordinate, then summed
  for (int it = tid; it < 2 * D; it += 256) {
    const int half = it / D, i = it - half * D;
    double acc = 0.0;
    for (int j = half; j < a.n_win; j += 2)
      acc = fma((double)sj[j], (double)wval(a.wv, base + (size_t)j * D + i), acc);
    po[half][i] = (float)acc;
  }
  __syncthreads();
  float *dst = a.wpart + (size_t)row * (2 + D);
  if (tid == 0) {
    dst[0] = M;
    dst[1] = (red[0] + red[1]) + (red[2] + red[3]);
  }
  for (int i = tid; i < D; i += 256) dst[2 + i] = po[0][i] + po[1][i];
}

// ---------------------------------------------------------------------------
// Multi-query (chunked-prefill) attention over the compressed cache ("Your KV
// cache is not a bit problem but a geometry problem", "Systems tax": a prompt
// chunk is appended along the token axis, then its queries read the cache).
// Each query row (query token i, head g of a KV head) attends to slots
// [0, n_ctx), or [0, min(n_ctx, q_pos0 + i + 1)) when causal.  The scan is a
// tile contraction on fp32 MFMA (v_mfma_f32_16x16x4_f32: exact fp32 products,
// fp32 sums).  A block owns 64 rows of one (b, KV head); each wave 16 rows.
// Per 16-token block a wave forms S^T = K^ Q'^T (M = tokens, N = rows, K =
// coordinates; A = centroids looked up from the LDS-staged codes, B = q' held
// in registers), so lane l holds the base-2 logits of row l%16 for tokens
// 4 (l/16) .. 4 (l/16) + 3; the online softmax runs on those registers, and the
// same registers are the A operand of O' += P V^ (one MFMA per token of the
// four: the contraction index of MFMA r is token 4 (l/16) + r), with
// c = p n_v folded into A and B = C_V[code].  The V sketch term accumulates
// a += (c rho_v) (2 sigma - 1) the same way.  Rows are finished by
// finish_kernel (S^T a, inverse rotation).
// ---------------------------------------------------------------------------
template <int BITS>
__device__ __forceinline__ uint32_t kcode_at(const uint32_t *w, int kk, int g, int dwords2) {
  // coordinate c = 4 kk + g of a record image (layout as in place_code)
  if constexpr (BITS == 4) return (w[kk >> 1] >> (16 * (kk & 1) + 4 * g)) & 15u;
  if constexpr (BITS == 2) return (w[kk >> 2] >> (8 * (kk & 3) + 2 * g)) & 3u;
  if constexpr (BITS == 1) return (w[kk >> 3] >> (4 * (kk & 7) + g)) & 1u;
  const uint32_t lo = (w[kk >> 2] >> (8 * (kk & 3) + 2 * g)) & 3u;
  const uint32_t hi = (w[dwords2 + (kk >> 3)] >> (4 * (kk & 7) + g)) & 1u;
  return lo | (hi << 2);
}
template <int BITS>
__device__ __forceinline__ uint32_t vcode_at(const uint32_t *w, int cb, int j, int dwords2) {
  // coordinate c = 16 cb + j
  if constexpr (BITS == 4) {
    // word 2 cb + (j >= 8), chosen by a mask (a selected array index would
    // send the record image to scratch)
    const uint32_t m = 0u - (uint32_t)(j >> 3);
    const uint32_t x = (w[2 * cb + 1] & m) | (w[2 * cb] & ~m);
    return (x >> (4 * (j & 7))) & 15u;
  }
  if constexpr (BITS == 2) return (w[cb] >> (2 * j)) & 3u;
  if constexpr (BITS == 1) return (w[cb >> 1] >> (16 * (cb & 1) + j)) & 1u;
  const uint32_t lo = (w[cb] >> (2 * j)) & 3u;
  const uint32_t hi = (w[dwords2 + (cb >> 1)] >> (16 * (cb & 1) + j)) & 1u;
  return lo | (hi << 2);
}

// Copy ntok records of rb bytes (2-byte multiples, contiguous in memory) into
// LDS rows of pitch `pitch` bytes, with halfword accesses (records are 2-byte
// aligned); all 256 threads.
__device__ __forceinline__ void stage_records(unsigned char *dst, int pitch, const uint8_t *src,
                                              int rb, int ntok, int tid) {
  const int nh = ntok * rb / 2;
  const uint16_t *s16 = (const uint16_t *)src;
  for (int k = tid; k < nh; k += 256) {
    const int t = (2 * k) / rb, off = 2 * k - t * rb;
    *(uint16_t *)(dst + t * pitch + off) = s16[k];
  }
}

template <int D, int KB, bool KQ, int VB, bool VQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D > 128 ? 1 : 2, D > 128 ? 1 : 2)))
void prefill_kernel(const PrefillArgs a) {
  constexpr int TT = 64;                              // tokens per staged tile
  constexpr int KBYTES = D * KB / 8, VBYTES = D * VB / 8, SBYTES = D / 8;
  constexpr int SP = (SBYTES + 15) / 16 * 16, SW = SP / 4;
  constexpr int KWR = (KBYTES + 3) / 4, VWR = (VBYTES + 3) / 4;
  constexpr int NKK = D / 4, NCB = D / 16;
  constexpr int KROW = NKK + 4;                       // padded row of the K tile
  // Dequantised tiles, laid out for the MFMA operand reads:
  //   kh_s[t][g][kk] = C_K[code_t(4 kk + g)]   (A of S^T: lane reads 4 kk at once)
  //   vh_s[t][j][cb] = C_V[code_t(16 cb + j)]  (B of P V: lane reads 4 cb at once)
  __shared__ __attribute__((aligned(16))) float kh_s[TT * 4 * KROW];
  __shared__ __attribute__((aligned(16))) float vh_s[TT * 16 * NCB];
  __shared__ __attribute__((aligned(16))) unsigned char ks_s[KQ ? TT * SP : 16];
  __shared__ __attribute__((aligned(16))) unsigned char vs_s[VQ ? TT * SP : 16];
  // value codes at d = 128 are stored in token groups: the tile's groups are
  // staged raw and read with vg_code
  constexpr bool VGR = D == 128;
  __shared__ __attribute__((aligned(16))) uint8_t vq_s[VGR ? TT * VBYTES : 16];
  __shared__ __attribute__((aligned(16))) float kn_s[TT], kr_s[TT], vn_s[TT], vr_s[TT];
  __shared__ float kct_s[16], vct_s[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, j = lane & 15;
  const int hkv = blockIdx.y, b = blockIdx.z;
  const size_t unit = (size_t)b * a.Hkv + hkv;
  const int NR = a.nq * a.G;
  const int rt = blockIdx.x / a.splits, split = blockIdx.x - rt * a.splits;
  const int R0 = rt * 64 + wave * 16;                 // first row of this wave
  const int t_lo = (a.t0 & ~15) + split * a.tps;      // this block's slots [t_lo, t_lo + tps)
  if (tid < 16) {
    kct_s[tid] = a.kcent[tid];
    vct_s[tid] = a.vcent[tid];
  }
  auto t_limit = [&](int R) {
    if (!a.causal) return a.n_ctx;
    const int lim = a.q_pos0 + R / a.G + 1;
    return lim < a.n_ctx ? lim : a.n_ctx;
  };
  const int Rj = R0 + j;
  // visible slots end at the row's limit and at this split's end
  const int tl = Rj < NR ? min(t_limit(Rj), t_lo + a.tps) : 0;
  const int tl_w = min(t_lo + a.tps, R0 < NR ? t_limit(min(R0 + 15, NR - 1)) : 0);
  const int tl_b = min(t_lo + a.tps, t_limit(min(rt * 64 + 63, NR - 1)));

  float qB[NKK], sqB[KQ ? NKK : 1];
  {
    const float *qrow = a.qt + (unit * NR + (Rj < NR ? Rj : 0)) * D;
    const float *sqrow = KQ ? a.sqt + (unit * NR + (Rj < NR ? Rj : 0)) * D : nullptr;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qB[kk] = Rj < NR ? qrow[4 * kk + g4] : 0.0f;
      if constexpr (KQ) sqB[kk] = Rj < NR ? sqrow[4 * kk + g4] : 0.0f;
    }
  }
  f32x4v acc_o[NCB], acc_a[VQ ? NCB : 1];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    acc_o[cb] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (VQ) acc_a[cb] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
  }
  float M = -INFINITY, L = 0.0f;                      // row j (replicated over g4)
  // dequantisation role of this thread: token dt, quarter dq
  const int dt = tid & (TT - 1), dq = tid >> 6;

  __syncthreads();                                    // centroid tables
  for (int tbase = t_lo; tbase < tl_b; tbase += TT) {
    const int ntok = min(TT, tl_b - tbase);
    const size_t rec0 = unit * a.cap + tbase;
    __syncthreads();                                  // previous tile consumed
    if constexpr (VGR) {
      // whole 16-slot blocks of the tile (the capacity is a multiple of 16)
      const int nb16 = (ntok + 15) / 16 * 16 * VBYTES / 16;
      const uint8_t *src = a.vc + rec0 * VBYTES;
      for (int k = tid; k < nb16; k += 256) *(u32x4 *)(vq_s + 16 * k) = *(const u32x4 *)(src + 16 * k);
      __syncthreads();
    }
    {
      // K: this thread's quarter g = dq of token dt, every kk
      const bool ok = dt < ntok;
      uint32_t kw[KWR + 1];
      kw[KWR] = 0u;
      if (ok) load_rec<KBYTES>(a.kc + (rec0 + dt) * KBYTES, kw);
      float *kd = kh_s + (dt * 4 + dq) * KROW;
#pragma unroll
      for (int q4 = 0; q4 < NKK / 4; ++q4) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = ok ? kct_s[kcode_at<KB>(kw, 4 * q4 + e, dq, D / 16)] : 0.0f;
        *(float4 *)(kd + 4 * q4) = float4{v[0], v[1], v[2], v[3]};
      }
      // V: lanes j = 4 dq .. 4 dq + 3 of token dt, every cb
      uint32_t vw[VWR + 1];
      vw[VWR] = 0u;
      if (!VGR && ok) load_rec<VBYTES>(a.vc + (rec0 + dt) * VBYTES, vw);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int jv = 4 * dq + jj;
        float *vd = vh_s + (dt * 16 + jv) * NCB;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const uint32_t code = VGR ? vg_code<VB>(vq_s, (size_t)dt, 16 * cb + jv)
                                    : vcode_at<VB>(vw, cb, jv, D / 16);
          vd[cb] = ok ? vct_s[code] : 0.0f;
        }
      }
    }
    if constexpr (KQ) stage_records(ks_s, SP, a.ks + rec0 * SBYTES, SBYTES, ntok, tid);
    if constexpr (VQ) {
      if constexpr (VGR) {
        // sign octets -> per-slot records (the 8 x 8 transpose is its own inverse)
        const int nit = (ntok + 7) / 8 * 16;
        for (int it = tid; it < nit; it += 256) {
          const int o = it >> 4, n = it & 15;
          const u32x2 w = *(const u32x2 *)(a.vs + rec0 * SBYTES + o * 128 + 8 * n);
          uint32_t lo = w.x, hi = w.y;
          vg_transpose8(lo, hi);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            vs_s[(8 * o + e) * SP + n] = (uint8_t)(((e < 4 ? lo : hi) >> (8 * (e & 3))) & 255u);
        }
      } else {
        stage_records(vs_s, SP, a.vs + rec0 * SBYTES, SBYTES, ntok, tid);
      }
    }
    if (tid < TT) {
      const bool ok = tid < ntok;
      kn_s[tid] = ok ? f16_bits_to_f32(a.kn[rec0 + tid]) : 0.0f;
      vn_s[tid] = ok ? f16_bits_to_f32(a.vn[rec0 + tid]) : 0.0f;
      kr_s[tid] = (KQ && ok) ? f16_bits_to_f32(a.kr[rec0 + tid]) : 0.0f;
      vr_s[tid] = (VQ && ok) ? f16_bits_to_f32(a.vr[rec0 + tid]) : 0.0f;
    }
    __syncthreads();
    // scores S^T[token 4 g4 + r][row j] of token block tb (and QKQV's sketch term)
    auto scores = [&](int tb, f32x4v &sc, f32x4v &sk) {
      sk = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
      {
        const int ta = 16 * tb + j;                   // A-operand token (local index)
        const float *kr = kh_s + (ta * 4 + g4) * KROW;
        // four independent accumulation chains (dependent MFMAs would wait
        // for each other's results)
        f32x4v c4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) c4[u] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int q4 = 0; q4 < NKK / 4; ++q4) {
          const float4 av = *(const float4 *)(kr + 4 * q4);
          c4[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, qB[4 * q4], c4[0], 0, 0, 0);
          c4[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, qB[4 * q4 + 1], c4[1], 0, 0, 0);
          c4[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, qB[4 * q4 + 2], c4[2], 0, 0, 0);
          c4[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, qB[4 * q4 + 3], c4[3], 0, 0, 0);
        }
        sc = (c4[0] + c4[1]) + (c4[2] + c4[3]);
        if constexpr (KQ) {
          uint32_t sw[SW];
#pragma unroll
          for (int q = 0; q < SW / 4; ++q) {
            const u32x4 v = *(const u32x4 *)(ks_s + ta * SP + 16 * q);
            sw[4 * q] = v.x; sw[4 * q + 1] = v.y; sw[4 * q + 2] = v.z; sw[4 * q + 3] = v.w;
          }
          f32x4v k2[2] = {f32x4v{0.0f, 0.0f, 0.0f, 0.0f}, f32x4v{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) {
            const float sg = ((sw[kk >> 3] >> (4 * (kk & 7) + g4)) & 1u) ? 1.0f : -1.0f;
            k2[kk & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(sg, sqB[kk], k2[kk & 1], 0, 0, 0);
          }
          sk = k2[0] + k2[1];
        }
      }
    };
    // blocks of this tile that some row of the wave can see
    const int nb = tl_w > tbase ? min(TT / 16, (tl_w - tbase + 15) / 16) : 0;
#pragma unroll 1
    for (int tb = 0; tb < nb; ++tb) {
      f32x4v sc, sk;
      scores(tb, sc, sk);
      const int tr0 = 16 * tb + 4 * g4;               // local token of register r = 0
      const float4 knv = *(const float4 *)(kn_s + tr0);
      const float4 vnv = *(const float4 *)(vn_s + tr0);
      const float kn4[4] = {knv.x, knv.y, knv.z, knv.w};
      const float vn4[4] = {vnv.x, vnv.y, vnv.z, vnv.w};
      float kr4[4] = {0.0f, 0.0f, 0.0f, 0.0f}, vr4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (KQ) {
        const float4 v = *(const float4 *)(kr_s + tr0);
        kr4[0] = v.x; kr4[1] = v.y; kr4[2] = v.z; kr4[3] = v.w;
      }
      if constexpr (VQ) {
        const float4 v = *(const float4 *)(vr_s + tr0);
        vr4[0] = v.x; vr4[1] = v.y; vr4[2] = v.z; vr4[3] = v.w;
      }
      // ---- online softmax (base 2) over the 16 tokens, row j ----
      float s[4], p[4];
      float mloc = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = sc[r];
        if constexpr (KQ) v = fmaf(a.kcoef * kr4[r], sk[r], v);
        v = kn4[r] * v;
        s[r] = (tbase + tr0 + r < tl && tbase + tr0 + r >= a.t0) ? v : -INFINITY;
        mloc = fmaxf(mloc, s[r]);
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      const float Mn = fmaxf(M, mloc);
      const float alpha = (Mn == -INFINITY) ? 1.0f : fast_exp2(M - Mn);
      float ps = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = (s[r] == -INFINITY) ? 0.0f : fast_exp2(s[r] - Mn);
        ps += p[r];
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      L = fmaf(alpha, L, ps);
      M = Mn;
      // rescale the accumulators (rows 4 g4 + rr) unless no row's max moved
      if (__ballot(alpha != 1.0f)) {
        float al[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) al[rr] = __shfl(alpha, 4 * g4 + rr, 64);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            acc_o[cb][rr] *= al[rr];
            if constexpr (VQ) acc_a[cb][rr] *= al[rr];
          }
      }
      // ---- O' += P V^, a += P (rho_v sign) ----
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tv = tr0 + r;                       // this lane's token for MFMA r
        const float c = p[r] * vn4[r];
        const float *vr = vh_s + (tv * 16 + j) * NCB;
        float bv[NCB];
        if constexpr (NCB >= 4) {
#pragma unroll
          for (int q4 = 0; q4 < NCB / 4; ++q4) {
            const float4 v = *(const float4 *)(vr + 4 * q4);
            bv[4 * q4] = v.x; bv[4 * q4 + 1] = v.y; bv[4 * q4 + 2] = v.z; bv[4 * q4 + 3] = v.w;
          }
        } else {
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) bv[cb] = vr[cb];
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          acc_o[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(c, bv[cb], acc_o[cb], 0, 0, 0);
        if constexpr (VQ) {
          const float cq = c * vr4[r];
          uint32_t sw[SW];
#pragma unroll
          for (int q = 0; q < SW / 4; ++q) {
            const u32x4 v = *(const u32x4 *)(vs_s + tv * SP + 16 * q);
            sw[4 * q] = v.x; sw[4 * q + 1] = v.y; sw[4 * q + 2] = v.z; sw[4 * q + 3] = v.w;
          }
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const float sg = ((sw[cb >> 1] >> (16 * (cb & 1) + j)) & 1u) ? 1.0f : -1.0f;
            acc_a[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(cq, sg, acc_a[cb], 0, 0, 0);
          }
        }
      }
    }
  }
  // partials of rows 4 g4 + rr: M, L, o', a (a split that sees no slot of a
  // row leaves M = -inf, L = 0 and zero sums)
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int R = R0 + 4 * g4 + rr;
    const float Mr = __shfl(M, 4 * g4 + rr, 64);
    const float Lr = __shfl(L, 4 * g4 + rr, 64);
    if (R < NR) {
      float *dst = a.part + ((unit * NR + R) * a.splits + split) * (2 + 2 * D);
      if (j == 0) {
        dst[0] = Mr;
        dst[1] = Lr;
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        dst[2 + 16 * cb + j] = acc_o[cb][rr];
        if constexpr (VQ) dst[2 + D + 16 * cb + j] = acc_a[cb][rr];
      }
    }
  }
}

// Multi-query attention below d = 16, where the tile kernels' 16-coordinate
// blocks do not fit: the same split partials (M, L, o', a) as prefill_kernel
// for the same grid (64 query rows of one (b, KV head) and one token split per
// block).  Wave w takes the slots t_lo + w, t_lo + w + 4, ... of the split,
// one thread per row, with an online base-2 softmax over exact fp32 scores
// from the stored codes; the four waves' partials are merged through LDS.
template <int D, int KB, bool KQ, int VB, bool VQ>
__global__ __launch_bounds__(256) void prefill_small_kernel(const PrefillArgs a) {
  constexpr int NS = 2 + 2 * D;
  constexpr int KREC = D * KB / 8, VREC = D * VB / 8, SREC = D / 8;
  __shared__ float ps[4][64][NS];
  __shared__ float kct_s[16], vct_s[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.z, hkv = blockIdx.y;
  const size_t unit = (size_t)b * a.Hkv + hkv;
  const int NR = a.nq * a.G;
  const int rt = blockIdx.x / a.splits, split = blockIdx.x - rt * a.splits;
  const int R = rt * 64 + lane;
  const int t_lo = (a.t0 & ~15) + split * a.tps;
  if (tid < 16) {
    kct_s[tid] = a.kcent[tid];
    vct_s[tid] = a.vcent[tid];
  }
  __syncthreads();
  // visible slots of row R in this split: [max(t_lo, t0), min(limit, t_lo + tps))
  int lim = 0;
  if (R < NR) {
    lim = a.n_ctx;
    if (a.causal) lim = min(lim, a.q_pos0 + R / a.G + 1);
    lim = min(lim, t_lo + a.tps);
  }
  const int t_start = max(t_lo, a.t0);
  float q[D], sq[KQ ? D : 1];
  {
    const size_t r = unit * NR + (R < NR ? R : 0);
#pragma unroll
    for (int i = 0; i < D; ++i) {
      q[i] = a.qt[r * D + i];
      if constexpr (KQ) sq[i] = a.sqt[r * D + i];
    }
  }
  float M = -INFINITY, L = 0.0f, o[D], av[VQ ? D : 1];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    o[i] = 0.0f;
    if constexpr (VQ) av[i] = 0.0f;
  }
  for (int t = t_start + wave; t < lim; t += 4) {
    const size_t slot = unit * a.cap + (size_t)t;
    const uint8_t *kr = a.kc + slot * KREC;
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < D; ++i) acc = fmaf(q[i], kct_s[get_code<D, KB>(kr, i)], acc);
    const float nk = f16_bits_to_f32(a.kn[slot]);
    float s;
    if constexpr (KQ) {
      const uint8_t *sg = a.ks + slot * SREC;
      float sk = 0.0f;
#pragma unroll
      for (int i = 0; i < D; ++i) sk = fmaf(sq[i], ((sg[i >> 3] >> (i & 7)) & 1) ? 1.0f : -1.0f, sk);
      s = nk * fmaf(a.kcoef * f16_bits_to_f32(a.kr[slot]), sk, acc);
    } else {
      s = nk * acc;
    }
    const float Mn = fmaxf(M, s);
    const float al = M == -INFINITY ? 0.0f : fast_exp2(M - Mn);
    const float w = fast_exp2(s - Mn);
    L = fmaf(L, al, w);
    const float c = w * f16_bits_to_f32(a.vn[slot]);
    const uint8_t *vr = a.vc + slot * VREC;
#pragma unroll
    for (int i = 0; i < D; ++i) o[i] = fmaf(c, vct_s[get_code<D, VB>(vr, i)], o[i] * al);
    if constexpr (VQ) {
      const float cq = c * f16_bits_to_f32(a.vr[slot]);
      const uint8_t *sg = a.vs + slot * SREC;
#pragma unroll
      for (int k = 0; k < D; ++k)
        av[k] = fmaf(cq, ((sg[k >> 3] >> (k & 7)) & 1) ? 1.0f : -1.0f, av[k] * al);
    }
    M = Mn;
  }
  ps[wave][lane][0] = M;
  ps[wave][lane][1] = L;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    ps[wave][lane][2 + i] = o[i];
    ps[wave][lane][2 + D + i] = VQ ? av[i] : 0.0f;
  }
  __syncthreads();
  if (wave == 0 && R < NR) {
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) Mx = fmaxf(Mx, ps[w][lane][0]);
    float f[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) f[w] = ps[w][lane][0] == -INFINITY ? 0.0f : fast_exp2(ps[w][lane][0] - Mx);
    float *dst = a.part + ((unit * NR + R) * a.splits + split) * NS;
    dst[0] = Mx;
    for (int k = 1; k < NS; ++k) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) v = fmaf(f[w], ps[w][lane][k], v);
      dst[k] = v;
    }
  }
}

// Finish of multi-query rows, FR rows per block of 256 threads (S staged once
// per block in LDS):  o = R^T (o' + sqrt(pi/2)/m S^T a)  (o', a already / L).
// Thread t owns row t / (D/8) and coordinates 8 (t % (D/8)) .. + 7.
template <int D>
struct FinishShape {
  static constexpr int TPR = D / 8;                 // threads per row
  static constexpr int FR = 256 / TPR;              // rows per block
};

template <int D, int RK, bool VQ>
__global__ __launch_bounds__(256) void finish_kernel(const FinishArgs a) {
  constexpr int TPR = FinishShape<D>::TPR, FR = FinishShape<D>::FR;
  __shared__ __attribute__((aligned(16))) uint16_t S_s[VQ ? D * D : 8];
  __shared__ __attribute__((aligned(16))) float a_s[FR][D];
  __shared__ __attribute__((aligned(16))) float v_s[FR][D];
  const int tid = threadIdx.x;
  const int r = tid / TPR, i0 = 8 * (tid % TPR);
  const int NR = a.nq * a.G;
  const size_t ridx = (size_t)blockIdx.x * FR + r;
  const bool ok = ridx < (size_t)a.rows;
  if constexpr (VQ) {
    for (int k = tid; k < D * D / 8; k += 256)
      *(u32x4 *)(S_s + 8 * k) = *(const u32x4 *)(a.S + 8 * (size_t)k);
  }
  // log-sum-exp merge of the row's token splits (base 2), then / L
  float v[8] = {0, 0, 0, 0, 0, 0, 0, 0}, av[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float Mc = -INFINITY, Lc = 0.0f;                    // merged max and sum of the compressed part
  {
    constexpr int NS = 2 + 2 * D;
    const float *src = a.part + (ok ? ridx : 0) * a.splits * NS;
    float Mx = -INFINITY;
    for (int sp = 0; sp < a.splits; ++sp) Mx = fmaxf(Mx, src[sp * NS]);
    float Ls = 0.0f;
    for (int sp = 0; sp < a.splits; ++sp) {
      const float *ps = src + sp * NS;
      const float w = ps[0] == -INFINITY ? 0.0f : fast_exp2(ps[0] - Mx);
      Ls = fmaf(w, ps[1], Ls);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = fmaf(w, ps[2 + i0 + e], v[e]);
        if constexpr (VQ) av[e] = fmaf(w, ps[2 + D + i0 + e], av[e]);
      }
    }
    const float inv = (ok && Ls > 0.0f) ? 1.0f / Ls : 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] *= inv;
      av[e] *= inv;
    }
    Mc = Mx;
    Lc = Ls;
  }
  if constexpr (VQ) {
#pragma unroll
    for (int e = 0; e < 8; ++e) a_s[r][i0 + e] = av[e];
    __syncthreads();
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k = 0; k < D; ++k) {
      const u32x4 sw = *(const u32x4 *)(S_s + k * D + i0);
      const float ak = a_s[r][k];
      acc[0] = fmaf(bf16_lo(sw.x), ak, acc[0]); acc[1] = fmaf(bf16_hi(sw.x), ak, acc[1]);
      acc[2] = fmaf(bf16_lo(sw.y), ak, acc[2]); acc[3] = fmaf(bf16_hi(sw.y), ak, acc[3]);
      acc[4] = fmaf(bf16_lo(sw.z), ak, acc[4]); acc[5] = fmaf(bf16_hi(sw.z), ak, acc[5]);
      acc[6] = fmaf(bf16_lo(sw.w), ak, acc[6]); acc[7] = fmaf(bf16_hi(sw.w), ak, acc[7]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = fmaf(a.vcoef, acc[e], v[e]);
  }
  if constexpr (RK != RK_NONE) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v_s[r][i0 + e] = v[e];
    __syncthreads();
    if constexpr (RK == RK_WHT || RK == RK_RHT) {
      // butterflies over each row: D/2 pairs per row, FR rows, 256 threads
      for (int h = 1; h < D; h <<= 1) {
        for (int pi = tid; pi < FR * D / 2; pi += 256) {
          const int rr = pi / (D / 2), q = pi - rr * (D / 2);
          const int ii = (q / h) * 2 * h + (q % h);
          const float x = v_s[rr][ii], y = v_s[rr][ii + h];
          v_s[rr][ii] = x + y;
          v_s[rr][ii + h] = x - y;
        }
        __syncthreads();
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = i0 + e;
        float x = v_s[r][i] * a.oscale;
        if constexpr (RK == RK_RHT) x = ((a.rsign[i >> 5] >> (i & 31)) & 1u) ? -x : x;
        v[e] = x;
      }
    } else {                                            // RK_QR: o = Q^T v
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = dense_rotate_back<D>(a.Q, v_s[r], i0 + e);
    }
  }
  if (ok) {
    const size_t unit = ridx / NR;
    const int R = (int)(ridx - unit * NR);
    const int b = (int)(unit / a.Hkv), hkv = (int)(unit - (size_t)b * a.Hkv);
    const int tq = R / a.G, g = R - tq * a.G;
    const size_t orow = ((size_t)b * a.nq + tq) * a.Hq + hkv * a.G + g;
    if (a.wpart) {
      // full-precision window: one more log-sum-exp step in the original
      // space (v is the compressed part already divided by its sum)
      const float *wp = a.wpart + orow * (2 + D);
      const float mu = wp[0], m = fmaxf(Mc, mu);
      const float ac = (Mc == -INFINITY) ? 0.0f : fast_exp2(Mc - m);
      const float au = (mu == -INFINITY) ? 0.0f : fast_exp2(mu - m);
      const float den = ac * Lc + au * wp[1];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (ac * Lc * v[e] + au * wp[2 + i0 + e]) / den;
    }
    float *dst = a.out + orow * D + i0;
    *(float4 *)dst = float4{v[0], v[1], v[2], v[3]};
    *(float4 *)(dst + 4) = float4{v[4], v[5], v[6], v[7]};
  }
}

}  // namespace kvq

#include "kvq_scan.hpp"
#include "kvq_prefill16.hpp"

namespace kvq {

// ---------------------------------------------------------------------------
// Dispatchers (host).  Only the (bits, rotation, sketch) combinations that the
// three schemes produce are instantiated.
// ---------------------------------------------------------------------------
// Blocks of 256 threads of kernel `kern` that the current device holds at
// once (every CU at the kernel's occupancy); looked up once per kernel and
// device.  0 when the runtime cannot tell.
inline int resident_blocks(const void *kern) {
  static std::mutex mu;
  static std::map<std::pair<const void *, int>, int> known;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(kern, dev);
  const auto it = known.find(key);
  if (it != known.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0) != hipSuccess)
    return 0;
  const int n = cus * (per_cu > 0 ? per_cu : 1);
  known[key] = n;
  return n;
}

// Persistent-style encoder launch: each wave walks tiles with a stride of
// 4 * grid.  Encoders with a bucketize table run one round of resident
// blocks, so each block builds its table once for many tiles; the others two.
inline hipError_t launch_tiles(const void *kern, const QuantArgs &a, bool lut, hipStream_t s) {
  const int want = (a.total_tiles + 3) / 4;
  const int r = resident_blocks(kern);
  const int cap = (r > 0 ? r : 256) * (lut ? 1 : 2);
  const int grid = want < cap ? want : cap;
  QuantArgs arg = a;
  void *args[] = {&arg};
  return hipLaunchKernel(kern, dim3(grid), dim3(256), args, 0, s);
}

template <int D, int BITS, int RK, bool QJL>
hipError_t quantize_go(const QuantArgs &a, bool bf16, bool vg, hipStream_t s) {
  constexpr bool LUT = BucketTables<BITS, (D >= 16)>::LUT;
  // value sides (token groups at d = 128): unrotated without sketch, or
  // rotated with sketch
  constexpr bool VGOK = D == 128 && ((RK == RK_NONE) != QJL);
  if (vg && !VGOK) return hipErrorInvalidValue;
  auto go = [&](auto V) -> hipError_t {
    constexpr bool VG = decltype(V)::value;
    if constexpr (RK == RK_QR) {
      if (bf16) return launch_tiles((const void *)&quantize_dense_kernel<D, BITS, QJL, true, VG>, a, LUT, s);
      return launch_tiles((const void *)&quantize_dense_kernel<D, BITS, QJL, false, VG>, a, LUT, s);
    } else {
      if (bf16) return launch_tiles((const void *)&quantize_kernel<D, BITS, RK, QJL, true, VG>, a, LUT, s);
      return launch_tiles((const void *)&quantize_kernel<D, BITS, RK, QJL, false, VG>, a, LUT, s);
    }
  };
  if constexpr (VGOK) {
    if (vg) return go(std::true_type{});
  }
  return go(std::false_type{});
}

template <int D, int RK>
hipError_t quantize_rot(const QuantArgs &a, int bits, bool qjl, bool bf16, bool vg, hipStream_t s) {
  if (!qjl) {
    switch (bits) {
      case 2: return quantize_go<D, 2, RK, false>(a, bf16, vg, s);
      case 3: return quantize_go<D, 3, RK, false>(a, bf16, vg, s);
      case 4: return quantize_go<D, 4, RK, false>(a, bf16, vg, s);
    }
  } else {
    switch (bits) {
      case 1: return quantize_go<D, 1, RK, true>(a, bf16, vg, s);
      case 2: return quantize_go<D, 2, RK, true>(a, bf16, vg, s);
      case 3: return quantize_go<D, 3, RK, true>(a, bf16, vg, s);
    }
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_quantize(const QuantArgs &a, int bits, int rk, bool qjl, bool bf16, bool vg,
                           hipStream_t s) {
  switch (rk) {
    case RK_NONE:
      if (qjl) return hipErrorInvalidValue;
      switch (bits) {
        case 1: return quantize_go<D, 1, RK_NONE, false>(a, bf16, vg, s);
        case 2: return quantize_go<D, 2, RK_NONE, false>(a, bf16, vg, s);
        case 3: return quantize_go<D, 3, RK_NONE, false>(a, bf16, vg, s);
        case 4: return quantize_go<D, 4, RK_NONE, false>(a, bf16, vg, s);
      }
      return hipErrorInvalidValue;
    case RK_WHT: return quantize_rot<D, RK_WHT>(a, bits, qjl, bf16, vg, s);
    case RK_RHT: return quantize_rot<D, RK_RHT>(a, bits, qjl, bf16, vg, s);
    case RK_QR: return quantize_rot<D, RK_QR>(a, bits, qjl, bf16, vg, s);
  }
  return hipErrorInvalidValue;
}

template <int D, int BITS, int RK, bool QJL>
hipError_t dequant_go(const DequantArgs &a, int n, hipStream_t s) {
  hipLaunchKernelGGL((dequant_kernel<D, BITS, RK, QJL>), dim3(n), dim3(D), 0, s, a);
  return hipGetLastError();
}

template <int D, int RK>
hipError_t dequant_rot(const DequantArgs &a, int bits, bool qjl, int n, hipStream_t s) {
  if (!qjl) {
    switch (bits) {
      case 2: return dequant_go<D, 2, RK, false>(a, n, s);
      case 3: return dequant_go<D, 3, RK, false>(a, n, s);
      case 4: return dequant_go<D, 4, RK, false>(a, n, s);
    }
  } else {
    switch (bits) {
      case 1: return dequant_go<D, 1, RK, true>(a, n, s);
      case 2: return dequant_go<D, 2, RK, true>(a, n, s);
      case 3: return dequant_go<D, 3, RK, true>(a, n, s);
    }
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_dequantize(const DequantArgs &a, int bits, int rk, bool qjl, int n,
                             hipStream_t s) {
  switch (rk) {
    case RK_NONE:
      if (qjl) return hipErrorInvalidValue;
      switch (bits) {
        case 1: return dequant_go<D, 1, RK_NONE, false>(a, n, s);
        case 2: return dequant_go<D, 2, RK_NONE, false>(a, n, s);
        case 3: return dequant_go<D, 3, RK_NONE, false>(a, n, s);
        case 4: return dequant_go<D, 4, RK_NONE, false>(a, n, s);
      }
      return hipErrorInvalidValue;
    case RK_WHT: return dequant_rot<D, RK_WHT>(a, bits, qjl, n, s);
    case RK_RHT: return dequant_rot<D, RK_RHT>(a, bits, qjl, n, s);
    case RK_QR: return dequant_rot<D, RK_QR>(a, bits, qjl, n, s);
  }
  return hipErrorInvalidValue;
}

template <int D, int RK>
hipError_t prep_go(const PrepArgs &a, bool kq, bool bf16, hipStream_t s) {
  const dim3 g(a.rows), blk(D);
  if (kq) {
    if (bf16) hipLaunchKernelGGL((prep_kernel<D, RK, true, true>), g, blk, 0, s, a);
    else hipLaunchKernelGGL((prep_kernel<D, RK, true, false>), g, blk, 0, s, a);
  } else {
    if (bf16) hipLaunchKernelGGL((prep_kernel<D, RK, false, true>), g, blk, 0, s, a);
    else hipLaunchKernelGGL((prep_kernel<D, RK, false, false>), g, blk, 0, s, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_prep(const PrepArgs &a, int rk, bool kq, bool bf16, hipStream_t s) {
  switch (rk) {
    case RK_NONE: return kq ? hipErrorInvalidValue : prep_go<D, RK_NONE>(a, false, bf16, s);
    case RK_WHT: return prep_go<D, RK_WHT>(a, kq, bf16, s);
    case RK_RHT: return prep_go<D, RK_RHT>(a, kq, bf16, s);
    case RK_QR: return prep_go<D, RK_QR>(a, kq, bf16, s);
  }
  return hipErrorInvalidValue;
}

template <int D, int KB, bool KQ, int VB, bool VQ>
hipError_t decode_go(const DecodeArgs &a, int gt, int B, int stages, hipStream_t s) {
  const dim3 grid(a.splits, a.Hkv * a.HG, B), blk(256);
  if (stages & STAGE_SCAN) {
    if constexpr (D == 128) {
      // matrix-core scan (every scheme and head grouping at d = 128)
      hipLaunchKernelGGL((scan_kernel<KB, KQ, VB, VQ>), grid, blk, 0, s, a);
    } else {
      switch (gt) {
        case 1: hipLaunchKernelGGL((decode_kernel<D, KB, KQ, VB, VQ, 1>), grid, blk, 0, s, a); break;
        case 2: hipLaunchKernelGGL((decode_kernel<D, KB, KQ, VB, VQ, 2>), grid, blk, 0, s, a); break;
        case 4: hipLaunchKernelGGL((decode_kernel<D, KB, KQ, VB, VQ, 4>), grid, blk, 0, s, a); break;
        default: return hipErrorInvalidValue;
      }
    }
  }
  if (stages & STAGE_MERGE) hipLaunchKernelGGL((merge_kernel<D, VQ>), dim3(B * a.Hq), blk, 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode(const DecodeArgs &a, int kb, bool kq, int vb, bool vq, int gt, int B,
                         int stages, hipStream_t s) {
  if (!kq && !vq && kb == vb) {  // KV
    switch (kb) {
      case 1: return decode_go<D, 1, false, 1, false>(a, gt, B, stages, s);
      case 2: return decode_go<D, 2, false, 2, false>(a, gt, B, stages, s);
      case 3: return decode_go<D, 3, false, 3, false>(a, gt, B, stages, s);
      case 4: return decode_go<D, 4, false, 4, false>(a, gt, B, stages, s);
    }
  } else if (!kq && vq && vb == kb - 1) {  // KQV
    switch (kb) {
      case 2: return decode_go<D, 2, false, 1, true>(a, gt, B, stages, s);
      case 3: return decode_go<D, 3, false, 2, true>(a, gt, B, stages, s);
      case 4: return decode_go<D, 4, false, 3, true>(a, gt, B, stages, s);
    }
  } else if (kq && vq && kb == vb) {  // QKQV
    switch (kb) {
      case 1: return decode_go<D, 1, true, 1, true>(a, gt, B, stages, s);
      case 2: return decode_go<D, 2, true, 2, true>(a, gt, B, stages, s);
      case 3: return decode_go<D, 3, true, 3, true>(a, gt, B, stages, s);
    }
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_window(const WindowArgs &a, bool q_bf16, bool w_bf16, int rows, hipStream_t s) {
  const dim3 g(rows), blk(256);
  if (q_bf16) {
    if (w_bf16) hipLaunchKernelGGL((window_kernel<D, true, true>), g, blk, 0, s, a);
    else hipLaunchKernelGGL((window_kernel<D, true, false>), g, blk, 0, s, a);
  } else {
    if (w_bf16) hipLaunchKernelGGL((window_kernel<D, false, true>), g, blk, 0, s, a);
    else hipLaunchKernelGGL((window_kernel<D, false, false>), g, blk, 0, s, a);
  }
  return hipGetLastError();
}

template <int D, int KB, bool KQ, int VB, bool VQ>
hipError_t prefill_go(const PrefillArgs &a, int B, hipStream_t s) {
  const int NR = a.nq * a.G;
  const dim3 grid((NR + 63) / 64 * a.splits, a.Hkv, B), blk(256);
  if constexpr (D == 128)
    hipLaunchKernelGGL((prefill16_kernel<KB, KQ, VB, VQ>), grid, blk, 0, s, a);
  else if constexpr (D >= 16)
    hipLaunchKernelGGL((prefill_kernel<D, KB, KQ, VB, VQ>), grid, blk, 0, s, a);
  else
    hipLaunchKernelGGL((prefill_small_kernel<D, KB, KQ, VB, VQ>), grid, blk, 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_prefill(const PrefillArgs &a, int kb, bool kq, int vb, bool vq, int B,
                          hipStream_t s) {
  if (!kq && !vq && kb == vb) {  // KV
    switch (kb) {
      case 1: return prefill_go<D, 1, false, 1, false>(a, B, s);
      case 2: return prefill_go<D, 2, false, 2, false>(a, B, s);
      case 3: return prefill_go<D, 3, false, 3, false>(a, B, s);
      case 4: return prefill_go<D, 4, false, 4, false>(a, B, s);
    }
  } else if (!kq && vq && vb == kb - 1) {  // KQV
    switch (kb) {
      case 2: return prefill_go<D, 2, false, 1, true>(a, B, s);
      case 3: return prefill_go<D, 3, false, 2, true>(a, B, s);
      case 4: return prefill_go<D, 4, false, 3, true>(a, B, s);
    }
  } else if (kq && vq && kb == vb) {  // QKQV
    switch (kb) {
      case 1: return prefill_go<D, 1, true, 1, true>(a, B, s);
      case 2: return prefill_go<D, 2, true, 2, true>(a, B, s);
      case 3: return prefill_go<D, 3, true, 3, true>(a, B, s);
    }
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_finish(const FinishArgs &a, bool vq, int rows, hipStream_t s) {
  constexpr int FR = FinishShape<D>::FR;
  const dim3 g((rows + FR - 1) / FR), blk(256);
#define KVQ_FIN(R, V) hipLaunchKernelGGL((finish_kernel<D, R, V>), g, blk, 0, s, a)
  switch (a.rk) {
    case RK_NONE: if (vq) return hipErrorInvalidValue; KVQ_FIN(RK_NONE, false); break;
    case RK_WHT: if (vq) KVQ_FIN(RK_WHT, true); else KVQ_FIN(RK_WHT, false); break;
    case RK_RHT: if (vq) KVQ_FIN(RK_RHT, true); else KVQ_FIN(RK_RHT, false); break;
    case RK_QR: if (vq) KVQ_FIN(RK_QR, true); else KVQ_FIN(RK_QR, false); break;
    default: return hipErrorInvalidValue;
  }
#undef KVQ_FIN
  return hipGetLastError();
}

#define KVQ_INSTANTIATE(D)                                                                     \
  template hipError_t launch_quantize<D>(const QuantArgs &, int, int, bool, bool, bool,           \
                                         hipStream_t);                                          \
  template hipError_t launch_dequantize<D>(const DequantArgs &, int, int, bool, int,            \
                                           hipStream_t);                                        \
  template hipError_t launch_prep<D>(const PrepArgs &, int, bool, bool, hipStream_t);           \
  template hipError_t launch_decode<D>(const DecodeArgs &, int, bool, int, bool, int, int, int, \
                                       hipStream_t);                                            \
  template hipError_t launch_window<D>(const WindowArgs &, bool, bool, int, hipStream_t);     \
  template hipError_t launch_prefill<D>(const PrefillArgs &, int, bool, int, bool, int,        \
                                        hipStream_t);                                           \
  template hipError_t launch_finish<D>(const FinishArgs &, bool, int, hipStream_t);

}  // namespace kvq
