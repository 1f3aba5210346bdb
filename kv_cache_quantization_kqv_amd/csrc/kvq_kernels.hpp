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

#include "kvq_internal.hpp"

#ifndef KVQ_DECODE_E4
#define KVQ_DECODE_E4 8  // coordinates per lane when four query heads share a KV head
#endif

namespace kvq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
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
// For |u| the top 11 bits of its fp32 pattern (exponent and 3 mantissa bits)
// are monotone in |u| and cut [0, 2) into cells whose width is at most 1/8 of
// their lower end.  Consecutive positive thresholds of the tables used here
// are more than 9/8 apart, so a cell holds at most one of them (the host
// checks this for every table it builds).  cell_lo[idx] counts the positive
// thresholds below the cell; one exact comparison with the next threshold
// finishes the count.  With the table symmetric and the middle threshold 0:
//   u > 0 : code = K/2 + #{P_k <  |u|}
//   u <= 0: code = K/2 - 1 - #{P_k <= |u|}
// which equals #{thresholds < u} (ties go to the lower cell).
// ---------------------------------------------------------------------------
struct BucketTables {
  uint8_t cell_lo[1024];   // per 11-bit |u| prefix: positive thresholds below the cell
  float pos[9];            // positive thresholds, then +inf sentinels
  float cent[16];
};

template <int BITS>
__device__ void build_bucket_tables(BucketTables &bt, const float *thr, const float *cent, int tid,
                                    int nthreads) {
  constexpr int K2 = 1 << (BITS - 1);
  for (int i = tid; i < 1024; i += nthreads) {
    const float lo = __uint_as_float((uint32_t)i << 20);
    int c = 0;
    for (int k = 0; k + 1 < K2; ++k) c += (thr[K2 + k] < lo) ? 1 : 0;
    bt.cell_lo[i] = (uint8_t)c;
  }
  if (tid < 9) bt.pos[tid] = (tid + 1 < K2) ? thr[K2 + tid] : INFINITY;
  if (tid < 16) bt.cent[tid] = cent[tid];
}

template <int BITS>
__device__ __forceinline__ uint32_t bucketize_lut(float u, const BucketTables &bt) {
  constexpr int K2 = 1 << (BITS - 1);
  const float au = fabsf(u);
  const uint32_t idx = min(__float_as_uint(au) >> 20, 1023u);  // |u| <= 1 (1+ulp) in practice
  const uint32_t c = bt.cell_lo[idx];
  const float p = bt.pos[c];
  const uint32_t lt = c + (p < au ? 1u : 0u);              // #{P_k <  |u|}
  const uint32_t le = lt + (p == au ? 1u : 0u);            // #{P_k <= |u|}
  return u > 0.0f ? (uint32_t)K2 + lt : (uint32_t)(K2 - 1) - le;
}

// Value of the partner lane (lane ^ 1) through a DPP quad permute (no LDS).
__device__ __forceinline__ float xor1_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t xor1_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}

// Codes of DL consecutive coordinates packed at compile-time positions: widths
// 1, 2, 4 as one little-endian image; width 3 as a 2-bit plane image (DL/16
// words) followed by a 1-bit plane image (DL/32 words, at least one).
template <int DL, int BITS>
struct LocalCodes {
  static constexpr int NA = BITS == 3 ? DL / 16 : (DL * BITS + 31) / 32;
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

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Quantize-on-write.  Blocks of 4 waves share the bucketize tables and (sketch
// sides) the sketch matrix S, staged once in LDS with a padded row pitch; each
// wave then walks its own tiles.  A tile is VT consecutive tokens of one
// (b, h), each token owned by LPV lanes (LPV = 2 for D = 128, else 1), each
// lane holding DL = D/LPV consecutive coordinates in registers.  The tile is
// read with coalesced 16-B loads into a padded LDS stage; the next tile's loads
// are issued before the current one is processed.
// Butterfly stages h < DL run in registers; the last stage of a split vector is
// one exchange with the partner lane (lane ^ 1), and the pairwise sum of
// squares of a split vector is (left half sum) + (right half sum), which is the
// root of the same adjacent-pair tree.  Then u = y * (1/nu), bucketize, pack.
// Sketch sides write the bf16 residual halves back to the stage and form
// z = S r~ for the tile with v_mfma_f32_32x32x16_bf16 (fp32 accumulate).  A
// sign is taken from z when |z| exceeds a bound on the accumulation error of
// any summation order, D * 2^-22 * ||S_k|| * ||r~|| (+2^-100 for flushed
// denormals); otherwise the lane recomputes that row in fp64, ascending, which
// is the definition.
// ---------------------------------------------------------------------------
template <int D, int BITS, bool ROT, bool QJL, bool BF16>
__global__ __launch_bounds__(256) void quantize_kernel(const QuantArgs a) {
  constexpr int LPV = D > 64 ? 2 : 1;        // lanes per vector
  constexpr int DL = D / LPV;                // coordinates per lane
  constexpr int VT = 64 / LPV;               // vectors per tile
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int ROWB = D * ESZ;
  constexpr int PITCH = ROWB + 16;
  constexpr int CPR = ROWB / 16;             // 16-B chunks per row
  constexpr int NLD = VT * CPR / 64;         // chunks per lane
  constexpr int RECB = D * BITS / 8;
  constexpr int RECW = (RECB + 3) / 4;
  constexpr int NCT = (D + 31) / 32;
  constexpr int NRT = VT / 32;
  constexpr int P2 = D * 2 + 16;             // bf16 row pitch (residuals, S)
  constexpr int SBYTES = QJL ? D * P2 : 16;
  static_assert(VT * P2 <= VT * PITCH, "residual rows must fit the staging buffer");
  static_assert((VT * CPR) % 64 == 0, "tile copy must split evenly over the wave");
  __shared__ __attribute__((aligned(16))) unsigned char stage_all[4][VT * PITCH];
  __shared__ __attribute__((aligned(16))) unsigned char S_s[SBYTES];
  __shared__ BucketTables bt;
  __shared__ float rn_all[4][VT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned char *stage = stage_all[wave];
  float *rn_s = rn_all[wave];
  const int vrow = lane / LPV;               // token row of this lane in the tile
  const int half = lane % LPV;               // which coordinate half
  build_bucket_tables<BITS>(bt, a.thr, a.cent, tid, 256);
  if constexpr (QJL) {
    for (int i = tid; i < D * (D / 8); i += 256) {     // 16-B chunks of S
      const int r = i / (D / 8), c = i - r * (D / 8);
      *(u32x4 *)(S_s + r * P2 + c * 16) = *(const u32x4 *)(a.S + (size_t)r * D + c * 8);
    }
  }
  __syncthreads();

  // largest sketch row norm (fp32, rounded up), for the sign-certification bound
  float a_snmax = 0.0f;
  if constexpr (QJL) {
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
    a_snmax = mx;
  }

  const int tile0 = blockIdx.x * 4 + wave;
  const int tstride = gridDim.x * 4;
  u32x4 pf[NLD];
  auto fetch = [&](int tile) {
    const int bh = tile / a.tiles_per_bh;
    const int tt = tile - bh * a.tiles_per_bh;
    const int b = bh / a.H, h = bh - b * a.H;
    const int tbase = tt * VT;
    const int nvalid = min(VT, a.T - tbase);
    const unsigned char *src0 = (const unsigned char *)a.src +
        ((long long)b * a.sb + (long long)h * a.sh + (long long)tbase * a.st) * ESZ;
    const long long rstride = a.st * ESZ;
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int ci = lane + 64 * k;
      const int r = ci / CPR, cc = ci - r * CPR;
      pf[k] = u32x4{0u, 0u, 0u, 0u};
      if (r < nvalid) pf[k] = *(const u32x4 *)(src0 + r * rstride + cc * 16);
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
    const int tbase = tt * VT;
    const int nvalid = min(VT, a.T - tbase);

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
    if (next < a.total_tiles) fetch(next);

    if constexpr (ROT) {
      wht_inplace<DL>(y);
      if constexpr (LPV == 2) {
        // last stage: (y_i, y_{i+DL}) -> (y_i + y_{i+DL}, y_i - y_{i+DL}); the upper
        // lane forms partner + (-own), which is the same rounded difference.
        const uint32_t flip = half ? 0x80000000u : 0u;
#pragma unroll
        for (int i = 0; i < DL; ++i) {
          const float other = xor1_f(y[i]);
          y[i] = other + __uint_as_float(__float_as_uint(y[i]) ^ flip);
        }
      }
    }
    float ss = pairwise_sumsq<DL>(y);
    if constexpr (LPV == 2) {
      const float o = xor1_f(ss);
      ss = half ? (o + ss) : (ss + o);
    }
    const float nu = sqrtf(ss);
    const float rcp = nu == 0.0f ? 0.0f : 1.0f / nu;
    LocalCodes<DL, BITS> lc;
    lc.clear();
#pragma unroll
    for (int i = 0; i < DL; ++i) {
      const float u = y[i] * rcp;
      const uint32_t code = bucketize_lut<BITS>(u, bt);
      lc.put(i, code);
      if constexpr (QJL) y[i] = u - bt.cent[code];
      // keep at most 16 coordinates' table lookups in flight (register pressure)
      if ((i & 15) == 15) __builtin_amdgcn_sched_barrier(0);
    }
    const bool valid = vrow < nvalid;
    const size_t slot = (size_t)bh * a.cap + (size_t)(a.t0 + tbase + vrow);
    uint32_t rec[RECW];
    if constexpr (LPV == 2) {
      // each lane packed its own half; the lower lane joins the two images
      LocalCodes<DL, BITS> oth;
#pragma unroll
      for (int k = 0; k < LocalCodes<DL, BITS>::NA + LocalCodes<DL, BITS>::NB; ++k)
        oth.w[k] = xor1_u(lc.w[k]);
      join_halves<D, DL, BITS, RECW>(rec, lc, oth);
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
    if (valid && half == 0) {
      store_bytes<RECB>(a.codes + slot * RECB, rec);
      a.norm[slot] = f32_to_f16_bits(nu * a.scale);
    }

    if constexpr (QJL) {
      float rs = pairwise_sumsq<DL>(y);
      if constexpr (LPV == 2) {
        const float o = xor1_f(rs);
        rs = half ? (o + rs) : (rs + o);
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
      wave_sync();

      // z^T = S r~^T per 32-token block: A = S rows (sketch rows k), B = r~ rows
      // (tokens t).  Output register j of lane l is z[k][t] with
      // k = 32 ct + 8 (j/4) + 4 (l/32) + (j%4) and t = l%32, so a lane holds 16
      // of its token's sign bits per 32-row block and lane l^32 the other 16.
#pragma unroll 1
      for (int rt = 0; rt < NRT; ++rt) {
        const int t = rt * 32 + (lane & 31);                  // token row in the tile
        const float rbt = rn_s[t];
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
            u32x4 sv = *(const u32x4 *)(S_s + ks_row * P2 + k0 * 2);
            if (!kok) sv = u32x4{0u, 0u, 0u, 0u};
            const u32x4 rv = *(const u32x4 *)(stage + t * P2 + k0 * 2);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, sv),
                                                          __builtin_bit_cast(bf16x8, rv), acc, 0,
                                                          0, 0);
          }
          // certified signs; uncertain entries are recomputed in fp64, ascending
          const float bound = fmaf(a_snmax, rbt, 0x1p-100f);
          uint32_t bits = 0u, unsure = 0u;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int bp = 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);   // bit = sketch row % 32
            const float z = acc[j];
            bits |= (z > 0.0f ? 1u : 0u) << bp;
            unsure |= (!(fabsf(z) > bound) ? 1u : 0u) << bp;
          }
          if constexpr (D < 32) unsure &= (1u << D) - 1u;                 // rows >= D do not exist
          if (t >= nvalid) unsure = 0u;                                    // padding rows of the tile
          while (unsure) {
            const int bp = __builtin_ctz(unsure);
            unsure &= unsure - 1u;
            const int k = ct * 32 + bp;
            const unsigned char *rr = stage + t * P2;
            const unsigned char *sr = S_s + k * P2;
            double sum = 0.0;
            for (int c = 0; c < D / 8; ++c) {
              const u32x4 rv = *(const u32x4 *)(rr + c * 16);
              const u32x4 sw4 = *(const u32x4 *)(sr + c * 16);
              const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
              const uint32_t sw[4] = {sw4.x, sw4.y, sw4.z, sw4.w};
#pragma unroll
              for (int k2 = 0; k2 < 4; ++k2) {
                sum = sum + (double)bf16_lo(sw[k2]) * (double)bf16_lo(rw[k2]);
                sum = sum + (double)bf16_hi(sw[k2]) * (double)bf16_hi(rw[k2]);
              }
            }
            bits = (bits & ~(1u << bp)) | ((sum >= 0.0 ? 1u : 0u) << bp);
          }
          sgw[ct] = bits | (uint32_t)__shfl_xor((int)bits, 32, 64);
        }
        const bool tvalid = t < nvalid && lane < 32;
        if (tvalid) {
          const size_t tslot = (size_t)bh * a.cap + (size_t)(a.t0 + tbase + t);
          uint8_t *dst = a.signs + tslot * (D / 8);
          if constexpr (D == 128) {
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
    wave_sync();
    if (next < a.total_tiles) stash();
    wave_sync();
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

// ---------------------------------------------------------------------------
// Dequantize (parity aid): one block of D threads per record.
//   x^ = ||x|| (H/sqrt(d)) (C[code] + sqrt(pi/2)/m ||r|| S^T (2 sigma - 1))
// ---------------------------------------------------------------------------
template <int D, int BITS, bool ROT, bool QJL>
__global__ __launch_bounds__(D) void dequant_kernel(const DequantArgs a) {
  __shared__ float t_s[D];
  __shared__ float sg_s[D];
  const int v = blockIdx.x, i = threadIdx.x;
  const int bh = v / a.T, t = v - bh * a.T;
  const size_t slot = (size_t)bh * a.cap + (size_t)(a.t0 + t);
  float val = a.cent[get_code<D, BITS>(a.codes + slot * (D * BITS / 8), i)];
  if constexpr (QJL) {
    const uint8_t *sg = a.signs + slot * (D / 8);
    sg_s[i] = ((sg[i >> 3] >> (i & 7)) & 1) ? 1.0f : -1.0f;
    __syncthreads();
    float acc = 0.0f;
    for (int k = 0; k < D; ++k) acc = acc + bf16_to_f32(a.S[(size_t)k * D + i]) * sg_s[k];
    val = val + a.coef * f16_bits_to_f32(a.rnorm[slot]) * acc;
  }
  if constexpr (ROT) val = wht_block<D>(t_s, val) * a.oscale;
  a.out[((size_t)bh * a.T + t) * D + i] = f16_bits_to_f32(a.norm[slot]) * val;
}

// ---------------------------------------------------------------------------
// Query preparation: qs = H q * log2(e)/d (rotated schemes) or q * log2(e)/sqrt(d),
// and for sketched keys sq = S qs.  Rotating q once replaces rotating every key
// (H is symmetric and H H = d I); log2(e) lets the scan use exp2.
// ---------------------------------------------------------------------------
template <int D, bool ROT, bool KQ, bool BF16>
__global__ __launch_bounds__(D) void prep_kernel(const PrepArgs a) {
  __shared__ float t_s[D];
  const int row = blockIdx.x, i = threadIdx.x;
  float x = BF16 ? bf16_to_f32(((const uint16_t *)a.q)[(size_t)row * D + i])
                 : ((const float *)a.q)[(size_t)row * D + i];
  if constexpr (ROT) x = wht_block<D>(t_s, x);
  x = x * a.qscale;
  a.qs[(size_t)row * D + i] = x;
  if constexpr (KQ) {
    __syncthreads();
    t_s[i] = x;
    __syncthreads();
    float acc = 0.0f;
    for (int k = 0; k < D; ++k) acc = acc + bf16_to_f32(a.S[(size_t)i * D + k]) * t_s[k];
    a.sq[(size_t)row * D + i] = acc;
  }
}

// ---------------------------------------------------------------------------
// Decode scan: one block (4 waves) per (token split, KV head, head group,
// batch row).  The split is walked in tiles of TT = 64 tokens.  Every segment
// of a tile (K codes, V codes, sign bits, fp16 norms; each contiguous in HBM)
// is copied into LDS with coalesced 16-byte loads spread over the whole block;
// the next tile's chunks are loaded into registers while the current tile is
// consumed, so HBM latency overlaps the arithmetic.
// Inside a tile a token is spread over L = D/E lanes (E = 16 coordinates per
// lane, 8 when four query heads share the KV head), so a wave covers 64/L
// tokens per pass; every lane keeps its E-coordinate slice of the GT query
// heads' rotated query, value accumulator and (sketched values) sketch-space
// accumulator.  Scores: sum of q'_i C_K[code_i] over the slice, reduced across
// the L lanes with DPP; online softmax in base 2 with lazy rescaling (the
// running max moves only when a score exceeds it by more than 20, so weights
// stay below 2^20 and fp32 sums keep their relative precision).
// Values: o' += w ||v|| C_V[code]; sketch: a += w ||v|| ||r|| (2 sigma - 1).
// ---------------------------------------------------------------------------
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

template <int BITS>
__device__ __forceinline__ int slice_code(uint32_t w0, uint32_t w1, int e) {
  if constexpr (BITS == 4) return (int)(((e < 8 ? w0 : w1) >> (4 * (e & 7))) & 15u);
  if constexpr (BITS == 3) return (int)(((w0 >> (2 * e)) & 3u) | (((w1 >> e) & 1u) << 2));
  if constexpr (BITS == 2) return (int)((w0 >> (2 * e)) & 3u);
  return (int)((w0 >> e) & 1u);
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

// Byte layout of one tile of TT tokens in LDS: the record segments back to back.
template <int D, int KB, bool KQ, int VB, bool VQ, int TT>
struct TileLayout {
  static constexpr int KREC = D * KB / 8, VREC = D * VB / 8, SREC = D / 8;
  static constexpr int KC = 0;
  static constexpr int VC = KC + TT * KREC;
  static constexpr int KS = VC + TT * VREC;
  static constexpr int VS = KS + (KQ ? TT * SREC : 0);
  static constexpr int KN = VS + (VQ ? TT * SREC : 0);
  static constexpr int VN = KN + TT * 2;
  static constexpr int KR = VN + TT * 2;
  static constexpr int VR = KR + (KQ ? TT * 2 : 0);
  static constexpr int BYTES = VR + (VQ ? TT * 2 : 0);
  static constexpr int NCH = BYTES / 16;
  static_assert(BYTES % 16 == 0 && KC % 16 == 0 && VC % 16 == 0 && KS % 16 == 0 &&
                VS % 16 == 0 && KN % 16 == 0 && VN % 16 == 0 && KR % 16 == 0 && VR % 16 == 0,
                "tile segments must be 16-byte multiples");
};

template <int D, int KB, bool KQ, int VB, bool VQ, int GT>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeArgs a) {
  constexpr int E = (GT >= 4 && D >= 16) ? KVQ_DECODE_E4 : 16;  // coordinates per lane
  constexpr int L = D / E;
  constexpr int TW = 64 / L;
  constexpr int NS = 2 + 2 * D;
  constexpr int TT = 64;
  using TL = TileLayout<D, KB, KQ, VB, VQ, TT>;
  constexpr int NPT = (TL::NCH + 255) / 256;         // 16-B chunks per thread per tile
  constexpr int NPASS = TT / TW;                     // token passes per tile
  constexpr int NPW = (NPASS + 3) / 4;               // passes per wave
  __shared__ __attribute__((aligned(16))) uint8_t tile[TL::BYTES];
  __shared__ float kc_s[16], vc_s[16];
  __shared__ float wmax_s[4][GT];
  __shared__ float wst[4][GT][NS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane % L, slot = lane / L;
  const int split = blockIdx.x;
  const int hkv = blockIdx.y / a.HG, hg = blockIdx.y - (blockIdx.y / a.HG) * a.HG;
  const int b = blockIdx.z;
  const int hq0 = hkv * a.Gtot + hg * GT;
  if (tid < 16) {
    kc_s[tid] = a.kcent[tid];
    vc_s[tid] = a.vcent[tid];
  }

  // this thread's chunks of a tile: segment base (at token 0), bytes per token,
  // byte offset inside the tile's segment
  const size_t unit = (size_t)b * a.Hkv + hkv;
  const uint8_t *cbase[NPT];
  int crec[NPT], coff[NPT];
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const int byte = (tid + 256 * k) * 16;
    const uint8_t *base = nullptr;
    int rec = 1, start = 0;
    if (byte < TL::VC) { base = a.kc; rec = TL::KREC; start = TL::KC; }
    else if (byte < TL::KS) { base = a.vc; rec = TL::VREC; start = TL::VC; }
    else if (byte < TL::VS) { base = a.ks; rec = TL::SREC; start = TL::KS; }
    else if (byte < TL::KN) { base = a.vs; rec = TL::SREC; start = TL::VS; }
    else if (byte < TL::VN) { base = (const uint8_t *)a.kn; rec = 2; start = TL::KN; }
    else if (byte < TL::KR) { base = (const uint8_t *)a.vn; rec = 2; start = TL::VN; }
    else if (byte < TL::VR) { base = (const uint8_t *)a.kr; rec = 2; start = TL::KR; }
    else if (byte < TL::BYTES) { base = (const uint8_t *)a.vr; rec = 2; start = TL::VR; }
    cbase[k] = base ? base + unit * a.cap * (size_t)rec : nullptr;
    crec[k] = rec;
    coff[k] = byte - start;
  }

  float q[GT][E];
  float sqv[GT][E];
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    const float *qr = a.qs + ((size_t)b * a.Hq + hq0 + hh) * D + g * E;
    const float *sr = a.sq + ((size_t)b * a.Hq + hq0 + hh) * D + g * E;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      q[hh][e] = qr[e];
      sqv[hh][e] = KQ ? sr[e] : 0.0f;
    }
  }
  // Block-uniform running max per head; per-lane partial sums (each token slot
  // adds its own tokens; slots and waves are summed at the end).
  float M[GT], Ls[GT], o[GT][E], av[GT][E];
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    M[hh] = -INFINITY;
    Ls[hh] = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      o[hh][e] = 0.0f;
      av[hh][e] = 0.0f;
    }
  }

  const int t_lo = split * a.tps;
  const int t_hi = min(a.n_ctx, t_lo + a.tps);
  const int ntiles = t_hi > t_lo ? (t_hi - t_lo + TT - 1) / TT : 0;
  u32x4 pf[NPT];
  auto fetch = [&](int it) {
    const int tt = t_lo + it * TT;
    const int nv = min(TT, t_hi - tt);
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      pf[k] = u32x4{0u, 0u, 0u, 0u};
      if (cbase[k] && coff[k] < nv * crec[k])
        pf[k] = *(const u32x4 *)(cbase[k] + (size_t)tt * crec[k] + coff[k]);
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int k = 0; k < NPT; ++k)
      if (cbase[k]) *(u32x4 *)(tile + (tid + 256 * k) * 16) = pf[k];
  };
  if (ntiles > 0) {
    fetch(0);
    stash();
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int nvalid = min(TT, t_hi - (t_lo + it * TT));
    if (it + 1 < ntiles) fetch(it + 1);

    // phase 1: scores of this wave's tokens of the tile (base-2 logits)
    float sct[NPW][GT];
#pragma unroll
    for (int pw = 0; pw < NPW; ++pw) {
      const int pass = wave + 4 * pw;
      const int tl = pass * TW + slot;
      const bool valid = pass < NPASS && tl < nvalid;
      const int tr = valid ? tl : 0;
      uint32_t kw0, kw1;
      lds_codes<D, KB, E>(tile + TL::KC + tr * TL::KREC, g, kw0, kw1);
      uint32_t ksg = 0u;
      if constexpr (KQ) {
        if constexpr (E == 16) ksg = *(const uint16_t *)(tile + TL::KS + tr * TL::SREC + g * 2);
        else ksg = tile[TL::KS + tr * TL::SREC + g];
      }
      const float nk = f16_bits_to_f32(*(const uint16_t *)(tile + TL::KN + tr * 2));
      const float rk = KQ ? f16_bits_to_f32(*(const uint16_t *)(tile + TL::KR + tr * 2)) : 0.0f;
      float sc[GT], sk[GT];
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) {
        sc[hh] = 0.0f;
        sk[hh] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float ck = kc_s[slice_code<KB>(kw0, kw1, e)];
#pragma unroll
        for (int hh = 0; hh < GT; ++hh) sc[hh] = fmaf(q[hh][e], ck, sc[hh]);
        if constexpr (KQ) {
          const float sg = ((ksg >> e) & 1u) ? 1.0f : -1.0f;
#pragma unroll
          for (int hh = 0; hh < GT; ++hh) sk[hh] = fmaf(sqv[hh][e], sg, sk[hh]);
        }
      }
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) {
        const float dot = group_sum<L>(sc[hh]);
        float s;
        if constexpr (KQ) s = nk * fmaf(a.kcoef * rk, group_sum<L>(sk[hh]), dot);
        else s = nk * dot;
        sct[pw][hh] = valid ? s : -INFINITY;
      }
    }
    // tile max per head: over this wave's passes and slots, then over the 4 waves
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      float m = sct[0][hh];
#pragma unroll
      for (int pw = 1; pw < NPW; ++pw) m = fmaxf(m, sct[pw][hh]);
#pragma unroll
      for (int off = L; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
      if (lane == 0) wmax_s[wave][hh] = m;
    }
    __syncthreads();
    // new running max (uniform over the block) and one rescale of the sums
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      const float tm = fmaxf(fmaxf(wmax_s[0][hh], wmax_s[1][hh]), fmaxf(wmax_s[2][hh], wmax_s[3][hh]));
      const float mn = fmaxf(M[hh], tm);
      const float al = (M[hh] == -INFINITY) ? 0.0f : fast_exp2(M[hh] - mn);
      M[hh] = mn;
      Ls[hh] *= al;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        o[hh][e] *= al;
        if constexpr (VQ) av[hh][e] *= al;
      }
    }
    // phase 2: weights, value and sketch sums
#pragma unroll
    for (int pw = 0; pw < NPW; ++pw) {
      const int pass = wave + 4 * pw;
      const int tl = pass * TW + slot;
      const bool valid = pass < NPASS && tl < nvalid;
      const int tr = valid ? tl : 0;
      uint32_t vw0, vw1;
      lds_codes<D, VB, E>(tile + TL::VC + tr * TL::VREC, g, vw0, vw1);
      uint32_t vsg = 0u;
      if constexpr (VQ) {
        if constexpr (E == 16) vsg = *(const uint16_t *)(tile + TL::VS + tr * TL::SREC + g * 2);
        else vsg = tile[TL::VS + tr * TL::SREC + g];
      }
      const float nv = f16_bits_to_f32(*(const uint16_t *)(tile + TL::VN + tr * 2));
      const float rv = VQ ? f16_bits_to_f32(*(const uint16_t *)(tile + TL::VR + tr * 2)) : 0.0f;
      float c[GT], cq[GT];
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) {
        const float w = valid ? fast_exp2(sct[pw][hh] - M[hh]) : 0.0f;
        Ls[hh] += w;
        c[hh] = w * nv;
        cq[hh] = c[hh] * rv;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float cv = vc_s[slice_code<VB>(vw0, vw1, e)];
#pragma unroll
        for (int hh = 0; hh < GT; ++hh) o[hh][e] = fmaf(c[hh], cv, o[hh][e]);
        if constexpr (VQ) {
          const float sg = ((vsg >> e) & 1u) ? 1.0f : -1.0f;
#pragma unroll
          for (int hh = 0; hh < GT; ++hh) av[hh][e] = fmaf(cq[hh], sg, av[hh][e]);
        }
      }
    }
    __syncthreads();
    if (it + 1 < ntiles) stash();
    __syncthreads();
  }

  // the max is block-uniform, so slots and waves combine by plain sums
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
  // Ls is replicated over the L lanes of a slot: sum one lane per slot
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    float l = (g == 0) ? Ls[hh] : 0.0f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) l += __shfl_xor(l, off, 64);
    Ls[hh] = l;
  }
  if (slot == 0) {
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      if (g == 0) {
        wst[wave][hh][0] = M[hh];
        wst[wave][hh][1] = Ls[hh];
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        wst[wave][hh][2 + g * E + e] = o[hh][e];
        wst[wave][hh][2 + D + g * E + e] = VQ ? av[hh][e] : 0.0f;
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < GT * (2 * D + 1); idx += 256) {
    const int hh = idx / (2 * D + 1), k = idx - hh * (2 * D + 1);
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) acc += (k == 2 * D ? wst[w][hh][1] : wst[w][hh][2 + k]);
    float *dst = a.part + (((size_t)b * a.Hq + hq0 + hh) * a.splits + split) * NS;
    if (k == 2 * D) {
      dst[0] = wst[0][hh][0];
      dst[1] = acc;
    } else {
      dst[2 + k] = acc;
    }
  }
}

// ---------------------------------------------------------------------------
// Combine: merge the split partials of one (b, hq) (log-sum-exp in base 2),
// add the sketch term sqrt(pi/2)/m S^T a, rotate back with one WHT, divide by
// the softmax normaliser.
// ---------------------------------------------------------------------------
template <int D, bool ROT, bool VQ>
__global__ __launch_bounds__(D) void combine_kernel(const CombineArgs a) {
  constexpr int NS = 2 + 2 * D;
  __shared__ float a_s[D];
  __shared__ float t_s[D];
  const int row = blockIdx.x, i = threadIdx.x;
  const float *p = a.part + (size_t)row * a.splits * NS;
  float mx = -INFINITY;
  for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, p[(size_t)s * NS]);
  float Lsum = 0.0f, ov = 0.0f, sv = 0.0f;
  for (int s = 0; s < a.splits; ++s) {
    const float ms = p[(size_t)s * NS];
    const float al = (ms == -INFINITY) ? 0.0f : exp2f(ms - mx);
    Lsum += al * p[(size_t)s * NS + 1];
    ov += al * p[(size_t)s * NS + 2 + i];
    if constexpr (VQ) sv += al * p[(size_t)s * NS + 2 + D + i];
  }
  if constexpr (VQ) {
    a_s[i] = sv;
    __syncthreads();
    float acc = 0.0f;
    for (int k = 0; k < D; ++k) acc = acc + bf16_to_f32(a.S[(size_t)k * D + i]) * a_s[k];
    ov = ov + a.vcoef * acc;
  }
  if constexpr (ROT) ov = wht_block<D>(t_s, ov);
  a.out[(size_t)row * D + i] = ov * a.oscale / Lsum;
}

// ---------------------------------------------------------------------------
// Dispatchers (host).  Only the (bits, rotation, sketch) combinations that the
// three schemes produce are instantiated.
// ---------------------------------------------------------------------------
template <int D, int BITS, bool ROT, bool QJL>
hipError_t quantize_go(const QuantArgs &a, bool bf16, hipStream_t s) {
  // persistent-style grid: each wave walks tiles with a stride of 4 * grid
  const int want = (a.total_tiles + 3) / 4;
  const int grid = want < 2048 ? want : 2048;
  if (bf16)
    hipLaunchKernelGGL((quantize_kernel<D, BITS, ROT, QJL, true>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((quantize_kernel<D, BITS, ROT, QJL, false>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_quantize(const QuantArgs &a, int bits, bool rot, bool qjl, bool bf16,
                           hipStream_t s) {
  if (!rot && !qjl) {
    switch (bits) {
      case 1: return quantize_go<D, 1, false, false>(a, bf16, s);
      case 2: return quantize_go<D, 2, false, false>(a, bf16, s);
      case 3: return quantize_go<D, 3, false, false>(a, bf16, s);
      case 4: return quantize_go<D, 4, false, false>(a, bf16, s);
    }
  } else if (rot && !qjl) {
    switch (bits) {
      case 2: return quantize_go<D, 2, true, false>(a, bf16, s);
      case 3: return quantize_go<D, 3, true, false>(a, bf16, s);
      case 4: return quantize_go<D, 4, true, false>(a, bf16, s);
    }
  } else if (rot && qjl) {
    switch (bits) {
      case 1: return quantize_go<D, 1, true, true>(a, bf16, s);
      case 2: return quantize_go<D, 2, true, true>(a, bf16, s);
      case 3: return quantize_go<D, 3, true, true>(a, bf16, s);
    }
  }
  return hipErrorInvalidValue;
}

template <int D, int BITS, bool ROT, bool QJL>
hipError_t dequant_go(const DequantArgs &a, int n, hipStream_t s) {
  hipLaunchKernelGGL((dequant_kernel<D, BITS, ROT, QJL>), dim3(n), dim3(D), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dequantize(const DequantArgs &a, int bits, bool rot, bool qjl, int n,
                             hipStream_t s) {
  if (!rot && !qjl) {
    switch (bits) {
      case 1: return dequant_go<D, 1, false, false>(a, n, s);
      case 2: return dequant_go<D, 2, false, false>(a, n, s);
      case 3: return dequant_go<D, 3, false, false>(a, n, s);
      case 4: return dequant_go<D, 4, false, false>(a, n, s);
    }
  } else if (rot && !qjl) {
    switch (bits) {
      case 2: return dequant_go<D, 2, true, false>(a, n, s);
      case 3: return dequant_go<D, 3, true, false>(a, n, s);
      case 4: return dequant_go<D, 4, true, false>(a, n, s);
    }
  } else if (rot && qjl) {
    switch (bits) {
      case 1: return dequant_go<D, 1, true, true>(a, n, s);
      case 2: return dequant_go<D, 2, true, true>(a, n, s);
      case 3: return dequant_go<D, 3, true, true>(a, n, s);
    }
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_prep(const PrepArgs &a, bool rot, bool kq, bool bf16, hipStream_t s) {
  const dim3 g(a.rows), blk(D);
#define KVQ_PREP(R, K, B) hipLaunchKernelGGL((prep_kernel<D, R, K, B>), g, blk, 0, s, a)
  if (rot) {
    if (kq) { if (bf16) KVQ_PREP(true, true, true); else KVQ_PREP(true, true, false); }
    else { if (bf16) KVQ_PREP(true, false, true); else KVQ_PREP(true, false, false); }
  } else {
    if (bf16) KVQ_PREP(false, false, true); else KVQ_PREP(false, false, false);
  }
#undef KVQ_PREP
  return hipGetLastError();
}

template <int D, int KB, bool KQ, int VB, bool VQ>
hipError_t decode_go(const DecodeArgs &a, int gt, int B, hipStream_t s) {
  const dim3 grid(a.splits, a.Hkv * a.HG, B), blk(256);
  switch (gt) {
    case 1: hipLaunchKernelGGL((decode_kernel<D, KB, KQ, VB, VQ, 1>), grid, blk, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<D, KB, KQ, VB, VQ, 2>), grid, blk, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_kernel<D, KB, KQ, VB, VQ, 4>), grid, blk, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode(const DecodeArgs &a, int kb, bool kq, int vb, bool vq, int gt, int B,
                         hipStream_t s) {
  if (!kq && !vq && kb == vb) {  // KV
    switch (kb) {
      case 1: return decode_go<D, 1, false, 1, false>(a, gt, B, s);
      case 2: return decode_go<D, 2, false, 2, false>(a, gt, B, s);
      case 3: return decode_go<D, 3, false, 3, false>(a, gt, B, s);
      case 4: return decode_go<D, 4, false, 4, false>(a, gt, B, s);
    }
  } else if (!kq && vq && vb == kb - 1) {  // KQV
    switch (kb) {
      case 2: return decode_go<D, 2, false, 1, true>(a, gt, B, s);
      case 3: return decode_go<D, 3, false, 2, true>(a, gt, B, s);
      case 4: return decode_go<D, 4, false, 3, true>(a, gt, B, s);
    }
  } else if (kq && vq && kb == vb) {  // QKQV
    switch (kb) {
      case 1: return decode_go<D, 1, true, 1, true>(a, gt, B, s);
      case 2: return decode_go<D, 2, true, 2, true>(a, gt, B, s);
      case 3: return decode_go<D, 3, true, 3, true>(a, gt, B, s);
    }
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_combine(const CombineArgs &a, bool rot, bool vq, int rows, hipStream_t s) {
  const dim3 g(rows), blk(D);
  if (rot) {
    if (vq) hipLaunchKernelGGL((combine_kernel<D, true, true>), g, blk, 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<D, true, false>), g, blk, 0, s, a);
  } else {
    if (vq) hipLaunchKernelGGL((combine_kernel<D, false, true>), g, blk, 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<D, false, false>), g, blk, 0, s, a);
  }
  return hipGetLastError();
}

#define KVQ_INSTANTIATE(D)                                                                     \
  template hipError_t launch_quantize<D>(const QuantArgs &, int, bool, bool, bool, hipStream_t); \
  template hipError_t launch_dequantize<D>(const DequantArgs &, int, bool, bool, int,           \
                                           hipStream_t);                                        \
  template hipError_t launch_prep<D>(const PrepArgs &, bool, bool, bool, hipStream_t);          \
  template hipError_t launch_decode<D>(const DecodeArgs &, int, bool, int, bool, int, int,      \
                                       hipStream_t);                                            \
  template hipError_t launch_combine<D>(const CombineArgs &, bool, bool, int, hipStream_t);

}  // namespace kvq
