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

namespace kvq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

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
// Quantize-on-write.  One wave (64 lanes) per block; a tile is VT consecutive
// tokens of one (b, h), each token owned by LPV lanes (LPV = 2 for D = 128,
// else 1), each lane holding DL = D/LPV consecutive coordinates in registers.
// The tile is read with coalesced 16-B loads into LDS (padded rows).
// Butterfly stages h < DL run in registers; the last stage of a split vector is
// one exchange with the partner lane (lane ^ 1), and the pairwise sum of
// squares of a split vector is (left half sum) + (right half sum), which is the
// root of the same adjacent-pair tree.  Then u = y * (1/nu), bucketize, pack.
// Sketch sides write the bf16 residual halves back to LDS and form z = S r~ for
// the tile with v_mfma_f32_32x32x16_bf16 (fp32 accumulate).  A sign is taken
// from z when |z| exceeds a bound on the accumulation error of any summation
// order, D * 2^-22 * ||S_k|| * ||r~|| (+2^-100 for flushed denormals);
// otherwise the lane recomputes that row in fp64, ascending, which is the
// definition.
// ---------------------------------------------------------------------------
template <int D, int BITS, bool ROT, bool QJL, bool BF16>
__global__ __launch_bounds__(64) void quantize_kernel(const QuantArgs a) {
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
  constexpr int P2 = D * 2 + 16;
  static_assert(VT * P2 <= VT * PITCH, "residual rows must fit the staging buffer");
  static_assert((VT * CPR) % 64 == 0, "tile copy must split evenly over the wave");
  __shared__ __attribute__((aligned(16))) unsigned char stage[VT * PITCH];
  __shared__ float cent_s[16];
  __shared__ float rn_s[VT];
  __shared__ uint32_t sg_s[VT * NCT];

  const int lane = threadIdx.x;
  const int vrow = lane / LPV;               // token row of this lane in the tile
  const int half = lane % LPV;               // which coordinate half
  if (lane < 16) cent_s[lane] = a.cent[lane];
  uint32_t thr[15];
#pragma unroll
  for (int k = 0; k < 15; ++k) {
    uint32_t v = __float_as_uint(a.thr[k]);
    asm volatile("" : "+v"(v));
    thr[k] = v;
  }

  float snorm[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) snorm[ct] = 0.0f;
  if constexpr (QJL) {
#pragma unroll 1
    for (int ct = 0; ct < NCT; ++ct) {
      const int col = ct * 32 + (lane & 31);
      float s = 0.0f;
      if (col < D) {
        for (int i = 0; i < D; ++i) {
          const float v = bf16_to_f32(a.S[(size_t)col * D + i]);
          s = s + v * v;
        }
      }
      snorm[ct] = sqrtf(s) * (1.0f + 0x1p-12f);
    }
  }
  __syncthreads();

#pragma unroll 1
  for (int tile = blockIdx.x; tile < a.total_tiles; tile += gridDim.x) {
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
      u32x4 v = {0u, 0u, 0u, 0u};
      if (r < nvalid) v = *(const u32x4 *)(src0 + r * rstride + cc * 16);
      *(u32x4 *)(stage + r * PITCH + cc * 16) = v;
    }
    __syncthreads();

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
    __syncthreads();

    if constexpr (ROT) {
      wht_inplace<DL>(y);
      if constexpr (LPV == 2) {
        // last stage: (y_i, y_{i+DL}) -> (y_i + y_{i+DL}, y_i - y_{i+DL}); the upper
        // lane forms partner + (-own), which is the same rounded difference.
        const uint32_t flip = half ? 0x80000000u : 0u;
#pragma unroll
        for (int i = 0; i < DL; ++i) {
          const float other = __shfl_xor(y[i], 1, 64);
          y[i] = other + __uint_as_float(__float_as_uint(y[i]) ^ flip);
        }
      }
    }
    float ss = pairwise_sumsq<DL>(y);
    if constexpr (LPV == 2) {
      const float o = __shfl_xor(ss, 1, 64);
      ss = half ? (o + ss) : (ss + o);
    }
    const float nu = sqrtf(ss);
    const float rcp = nu == 0.0f ? 0.0f : 1.0f / nu;
    uint32_t rec[RECW];
#pragma unroll
    for (int w = 0; w < RECW; ++w) rec[w] = 0u;
#pragma unroll
    for (int i = 0; i < DL; ++i) {
      const float u = y[i] * rcp;
      const uint32_t code = bucketize<BITS>(u, thr);
      place_code<D, BITS>(rec, half * DL + i, code);
      if constexpr (QJL) y[i] = u - cent_s[code];
    }
    const bool valid = vrow < nvalid;
    const size_t slot = (size_t)bh * a.cap + (size_t)(a.t0 + tbase + vrow);
    if constexpr (LPV == 2) {
      // each lane built the codes of its half; merge the two word images
#pragma unroll
      for (int w = 0; w < RECW; ++w) rec[w] |= __shfl_xor(rec[w], 1, 64);
    }
    if (valid && half == 0) {
      store_bytes<RECB>(a.codes + slot * RECB, rec);
      a.norm[slot] = f32_to_f16_bits(nu * a.scale);
    }

    if constexpr (QJL) {
      float rs = pairwise_sumsq<DL>(y);
      if constexpr (LPV == 2) {
        const float o = __shfl_xor(rs, 1, 64);
        rs = half ? (o + rs) : (rs + o);
      }
      const float rho = sqrtf(rs);
      if (valid && half == 0) a.rnorm[slot] = f32_to_f16_bits(rho);
      float rt2 = 0.0f;
      unsigned char *rrow = stage + vrow * P2 + half * DL * 2;
#pragma unroll
      for (int c = 0; c < DL / 8; ++c) {
        uint32_t wv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t lo = f32_to_bf16_rne(y[8 * c + 2 * k]);
          const uint32_t hi = f32_to_bf16_rne(y[8 * c + 2 * k + 1]);
          const float flo = __uint_as_float(lo << 16), fhi = __uint_as_float(hi << 16);
          rt2 = rt2 + flo * flo;
          rt2 = rt2 + fhi * fhi;
          wv[k] = lo | (hi << 16);
        }
        *(u32x4 *)(rrow + c * 16) = u32x4{wv[0], wv[1], wv[2], wv[3]};
      }
      if constexpr (LPV == 2) rt2 = rt2 + __shfl_xor(rt2, 1, 64);
      if (half == 0) rn_s[vrow] = sqrtf(rt2) * (1.0f + 0x1p-12f);
      __syncthreads();

#pragma unroll 1
      for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll 1
        for (int ct = 0; ct < NCT; ++ct) {
          f32x16 acc;
#pragma unroll
          for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
          const int col = ct * 32 + (lane & 31);
          const bool colok = col < D;
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks) {
            const int k0 = ks * 16 + 8 * (lane >> 5);
            const u32x4 av = *(const u32x4 *)(stage + (rt * 32 + (lane & 31)) * P2 + k0 * 2);
            u32x4 bv = {0u, 0u, 0u, 0u};
            if (colok) bv = *(const u32x4 *)(a.S + (size_t)col * D + k0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                          __builtin_bit_cast(bf16x8, bv), acc, 0,
                                                          0, 0);
          }
          // sign bits from z where certified; rows left uncertain are redone in fp64
          uint32_t bits = 0u, unsure = 0u;
          const float sn = snorm[ct];
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int row = rt * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
            const float z = acc[j];
            const float bound = (float)D * 0x1p-22f * sn * rn_s[row] + 0x1p-100f;
            bits |= (z > 0.0f ? 1u : 0u) << j;
            unsure |= ((colok && !(fabsf(z) > bound)) ? 1u : 0u) << j;
          }
          while (unsure) {
            const int j = __builtin_ctz(unsure);
            unsure &= unsure - 1u;
            const int row = rt * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
            const uint16_t *rr = (const uint16_t *)(stage + row * P2);
            const uint16_t *sr = a.S + (size_t)col * D;
            double sum = 0.0;
            for (int i = 0; i < D; ++i)
              sum = sum + (double)bf16_to_f32(sr[i]) * (double)bf16_to_f32(rr[i]);
            bits = (bits & ~(1u << j)) | ((sum >= 0.0 ? 1u : 0u) << j);
          }
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int row = rt * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
            const unsigned long long m = __ballot((bits >> j) & 1u);
            if (lane == 0) sg_s[row * NCT + ct] = (uint32_t)m;
            if (lane == 32) sg_s[row * NCT + ct] = (uint32_t)(m >> 32);
          }
        }
      }
      __syncthreads();
      if (valid && half == 0) {
        uint8_t *dst = a.signs + slot * (D / 8);
        if constexpr (D == 128) {
          *(u32x4 *)dst = u32x4{sg_s[vrow * 4], sg_s[vrow * 4 + 1], sg_s[vrow * 4 + 2], sg_s[vrow * 4 + 3]};
        } else if constexpr (D == 64) {
          *(u32x2 *)dst = u32x2{sg_s[vrow * 2], sg_s[vrow * 2 + 1]};
        } else if constexpr (D == 32) {
          *(uint32_t *)dst = sg_s[vrow];
        } else {
          *(uint16_t *)dst = (uint16_t)(sg_s[vrow] & 0xFFFFu);
        }
      }
      __syncthreads();
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
// batch row).  A token is spread over L = D/16 lanes, 16 coordinates each, so a
// wave covers 64/L tokens per step; every lane keeps its 16-coordinate slice of
// the GT query heads' rotated query, value accumulator and (sketched values)
// sketch-space accumulator.  Scores: sum of q'_i C_K[code_i] over the slice,
// reduced across the L lanes; online softmax in base 2 with lazy rescaling
// (the running max moves only when a score exceeds it by more than 8).
// Values: o' += w ||v|| C_V[code]; sketch: a += w ||v|| ||r|| (2 sigma - 1).
// ---------------------------------------------------------------------------
// Load the codes of coordinates [g*E, g*E+E) of one record (E = 16 or 8).
template <int D, int BITS, int E>
__device__ __forceinline__ void load_codes(const uint8_t *base, size_t rec, int g, uint32_t &w0,
                                           uint32_t &w1) {
  constexpr int RB = D * BITS / 8;
  const uint8_t *r = base + rec * RB;
  if constexpr (E == 16) {
    if constexpr (BITS == 4) {
      const u32x2 v = *(const u32x2 *)(r + g * 8);
      w0 = v.x;
      w1 = v.y;
    } else if constexpr (BITS == 3) {
      if constexpr (RB % 4 == 0) {
        w0 = *(const uint32_t *)(r + g * 4);
      } else {  // 6-byte records (D = 16) are only 2-byte aligned
        w0 = (uint32_t)*(const uint16_t *)(r + g * 4) | ((uint32_t)*(const uint16_t *)(r + g * 4 + 2) << 16);
      }
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

template <int D, int KB, bool KQ, int VB, bool VQ, int GT>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeArgs a) {
  constexpr int E = (GT >= 4 && D >= 16) ? 8 : 16;  // coordinates per lane
  constexpr int L = D / E;
  constexpr int TW = 64 / L;
  constexpr int NS = 2 + 2 * D;
  __shared__ float kc_s[16], vc_s[16];
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
  float o[GT][E], av[GT][E], M[GT], Ls[GT];
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
  __syncthreads();

  const int t_lo = split * a.tps;
  const int t_hi = min(a.n_ctx, t_lo + a.tps);
  const size_t base = ((size_t)b * a.Hkv + hkv) * a.cap;
  for (int t0 = t_lo + wave * TW; t0 < t_hi; t0 += 4 * TW) {
    const int t = t0 + slot;
    const bool valid = t < t_hi;
    const size_t rec = base + (size_t)(valid ? t : t_lo);
    uint32_t kw0, kw1, vw0, vw1;
    load_codes<D, KB, E>(a.kc, rec, g, kw0, kw1);
    load_codes<D, VB, E>(a.vc, rec, g, vw0, vw1);
    uint32_t ksg = 0u, vsg = 0u;
    if constexpr (E == 16) {
      if constexpr (KQ) ksg = *(const uint16_t *)(a.ks + rec * (D / 8) + g * 2);
      if constexpr (VQ) vsg = *(const uint16_t *)(a.vs + rec * (D / 8) + g * 2);
    } else {
      if constexpr (KQ) ksg = a.ks[rec * (D / 8) + g];
      if constexpr (VQ) vsg = a.vs[rec * (D / 8) + g];
    }
    const float nk = f16_bits_to_f32(a.kn[rec]);
    const float nv = f16_bits_to_f32(a.vn[rec]);
    const float rk = KQ ? f16_bits_to_f32(a.kr[rec]) : 0.0f;
    const float rv = VQ ? f16_bits_to_f32(a.vr[rec]) : 0.0f;

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
    for (int off = 1; off < L; off <<= 1) {
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) {
        sc[hh] += __shfl_xor(sc[hh], off, 64);
        if constexpr (KQ) sk[hh] += __shfl_xor(sk[hh], off, 64);
      }
    }
    bool need = false;
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      float s = KQ ? nk * fmaf(a.kcoef * rk, sk[hh], sc[hh]) : nk * sc[hh];
      sc[hh] = valid ? s : -INFINITY;
      need = need || (sc[hh] > M[hh] + 8.0f);
    }
    if (__any(need)) {
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) {
        const float mn = (sc[hh] > M[hh] + 8.0f) ? sc[hh] : M[hh];
        const float al = (mn == M[hh]) ? 1.0f : exp2f(M[hh] - mn);
        Ls[hh] *= al;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          o[hh][e] *= al;
          if constexpr (VQ) av[hh][e] *= al;
        }
        M[hh] = mn;
      }
    }
    float c[GT], cq[GT];
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      const float w = valid ? exp2f(sc[hh] - M[hh]) : 0.0f;
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

  // merge the token slots of this wave (lanes with equal g)
#pragma unroll
  for (int off = L; off < 64; off <<= 1) {
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      const float M2 = __shfl_xor(M[hh], off, 64);
      const float L2 = __shfl_xor(Ls[hh], off, 64);
      const float mn = fmaxf(M[hh], M2);
      const float a1 = (M[hh] == mn) ? 1.0f : exp2f(M[hh] - mn);
      const float a2 = (M2 == mn) ? 1.0f : exp2f(M2 - mn);
      Ls[hh] = Ls[hh] * a1 + L2 * a2;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        o[hh][e] = o[hh][e] * a1 + __shfl_xor(o[hh][e], off, 64) * a2;
        if constexpr (VQ) av[hh][e] = av[hh][e] * a1 + __shfl_xor(av[hh][e], off, 64) * a2;
      }
      M[hh] = mn;
    }
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
  // merge the 4 waves and write this split's partial state
  for (int idx = tid; idx < GT * (2 * D + 1); idx += 256) {
    const int hh = idx / (2 * D + 1), k = idx - hh * (2 * D + 1);
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mx = fmaxf(mx, wst[w][hh][0]);
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = wst[w][hh][0];
      const float al = (mw == -INFINITY) ? 0.0f : exp2f(mw - mx);
      acc += al * (k == 2 * D ? wst[w][hh][1] : wst[w][hh][2 + k]);
    }
    float *dst = a.part + (((size_t)b * a.Hq + hq0 + hh) * a.splits + split) * NS;
    if (k == 2 * D) {
      dst[0] = mx;
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
  const int grid = a.total_tiles < 16384 ? a.total_tiles : 16384;
  if (bf16)
    hipLaunchKernelGGL((quantize_kernel<D, BITS, ROT, QJL, true>), dim3(grid), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((quantize_kernel<D, BITS, ROT, QJL, false>), dim3(grid), dim3(64), 0, s, a);
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
