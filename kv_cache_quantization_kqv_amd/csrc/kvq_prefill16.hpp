// kvq_prefill16.hpp -- multi-query (chunked-prefill) attention over the
// compressed cache on the fp16 matrix cores, head dimension 128.  Included by
// kvq_kernels.hpp.
//
// Same work split and partial layout as prefill_kernel: a block owns 64 query
// rows (row = i G + g) of one (b, KV head) and one token split; each wave owns
// 16 rows.  Per 64-token tile the block dequantises the cache once into LDS,
// as fp16 operands that every wave shares:
//   kt_s[t][c]   key centroid of token t, coordinate c   (A of the scores)
//   kp_s[t][k]   key sign spin +-1 (QKQV)                 (A of the key sketch)
//   vt_s[c][t]   value centroid, coordinate-major         (B of P V)
//   st_s[k][t]   value sign spin +-1                      (B of the value sketch)
// The codebook levels are binary16 values and spins are +-1, so these are
// exact.  The other operands are fp32 quantities carried as x = xh + 2^-11 xl
// (split_pair: xh = fp16(x), xl = fp16((x - xh) 2^11)), with separate accumulators for
// the two parts, combined as hi + lo / 2048: the prepared query q' (and S q')
// scaled per row by a power of two into fp16 range, and the weights c = p n_v
// and c rho_v.
//
// All contractions use v_mfma_f32_16x16x32_f16.  Scores of a 16-token block:
// D[token][row] = sum_k K^[token][k] q'[row][k], so lane l holds the base-2
// logits of row l % 16 for tokens 4 (l / 16) + r, r = 0..3.  Two blocks form
// one step of the online softmax, and the same lane then supplies the A
// operand of O' += P V^ for its row and the 8 tokens it holds (slot e of lane
// group g <-> token 4 g + e of the first block, 4 g + e - 4 of the second;
// the B operand reads V^ for exactly those tokens), so the probabilities
// never leave the registers.  Rows are finished by finish_kernel.
#pragma once

namespace kvq {

// Code of local coordinate i (0..31) of one quarter of a per-slot record
// (words of the quarter as loaded below; width 3: two words of the 2-bit
// plane, then the word of the 1-bit plane).
template <int KB>
__device__ __forceinline__ uint32_t quarter_code(const uint32_t *w, int i) {
  if constexpr (KB == 4) return (w[i >> 3] >> (4 * (i & 7))) & 15u;
  if constexpr (KB == 2) return (w[i >> 4] >> (2 * (i & 15))) & 3u;
  if constexpr (KB == 1) return (w[0] >> i) & 1u;
  return ((w[i >> 4] >> (2 * (i & 15))) & 3u) | (((w[2] >> i) & 1u) << 2);
}

// Code of slot r (0..3) of a quad at coordinate 8 n + j of the piece words w
// (token-group value layout).
template <int VB>
__device__ __forceinline__ uint32_t piece_code(const uint32_t *w, int j, int r) {
  auto byte = [&](int i) { return (w[i >> 2] >> (8 * (i & 3))) & 255u; };
  if constexpr (VB == 4) {
    return (byte(2 * j + (r >> 1)) >> (4 * (r & 1))) & 15u;
  } else if constexpr (VB == 3) {
    const int u = 2 * j + (r >> 1);
    uint32_t P;
    if (u < 12) {
      P = byte(u) >> 2;
    } else {
      const int m = u - 12;
      P = (byte(m) & 3u) | ((byte(4 + m) & 3u) << 2) | ((byte(8 + m) & 3u) << 4);
    }
    return (P >> (3 * (r & 1))) & 7u;
  } else if constexpr (VB == 2) {
    return (byte(j) >> (2 * r)) & 3u;
  } else {
    return (w[0] >> (4 * j + r)) & 1u;
  }
}

template <int KB, bool KQ, int VB, bool VQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill16_kernel(const PrefillArgs a) {
  constexpr int D = 128, TT = 64;
  constexpr int KBYTES = D * KB / 8, VBYTES = D * VB / 8;
  constexpr int KP = D + 8;                          // fp16 pitch of the token-major tiles
  constexpr int VP = TT + 8;                         // fp16 pitch of the coordinate-major tiles
  __shared__ __attribute__((aligned(16))) _Float16 kt_s[TT * KP];
  __shared__ __attribute__((aligned(16))) _Float16 kp_s[KQ ? TT * KP : 8];
  __shared__ __attribute__((aligned(16))) _Float16 vt_s[D * VP];
  __shared__ __attribute__((aligned(16))) _Float16 st_s[VQ ? D * VP : 8];
  __shared__ __attribute__((aligned(16))) float kn_s[TT], kr_s[TT], vn_s[TT], vr_s[TT];
  __shared__ _Float16 kc_s[16], vc_s[16];
  __shared__ __attribute__((aligned(8))) u32x2 sp_s[16];   // nibble -> 4 fp16 spins

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int hkv = blockIdx.y, b = blockIdx.z;
  const size_t unit = (size_t)b * a.Hkv + hkv;
  const int NR = a.nq * a.G;
  const int rt = blockIdx.x / a.splits, split = blockIdx.x - rt * a.splits;
  const int R0 = rt * 64 + wave * 16;                 // first row of this wave
  const int t_lo = (a.t0 & ~15) + split * a.tps;      // this block's slots [t_lo, t_lo + tps)
  if (tid < 16) {
    kc_s[tid] = (_Float16)a.kcent[tid];
    vc_s[tid] = (_Float16)a.vcent[tid];
    uint32_t w[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
      w[q] = (((tid >> (2 * q)) & 1) ? 0x3C00u : 0xBC00u) | ((((tid >> (2 * q + 1)) & 1) ? 0x3C00u : 0xBC00u) << 16);
    sp_s[tid] = u32x2{w[0], w[1]};
  }
  auto t_limit = [&](int R) {
    if (!a.causal) return a.n_ctx;
    const int lim = a.q_pos0 + R / a.G + 1;
    return lim < a.n_ctx ? lim : a.n_ctx;
  };
  const int Rj = R0 + n;                              // this lane's row (scores, softmax)
  const int tl = Rj < NR ? min(t_limit(Rj), t_lo + a.tps) : 0;
  const int tl_w = min(t_lo + a.tps, R0 < NR ? t_limit(min(R0 + 15, NR - 1)) : 0);
  const int tl_b = min(t_lo + a.tps, t_limit(min(rt * 64 + 63, NR - 1)));

  // ---- query operands: row n, coordinates 32 kb + 8 g + e, scaled by 2^kq ----
  f16x8 qh[4], ql[4], sh[KQ ? 4 : 1], sl[KQ ? 4 : 1];
  float unq = 0.0f, uns = 0.0f;
  auto load_q = [&](const float *src, f16x8 (&h)[4], f16x8 (&l)[4], float &unscale) {
    float v[32];
    float m = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[8 * kb + e] = Rj < NR ? src[32 * kb + 8 * g + e] : 0.0f;
        m = fmaxf(m, fabsf(v[8 * kb + e]));
      }
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    int ex = 0;
    const bool fin = m > 0.0f && m <= 3.0e38f;
    if (fin) (void)frexpf(m, &ex);
    const int k = fin ? 14 - ex : 0;                  // |q 2^k| < 2^14
    unscale = ldexpf(1.0f, -k);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        split_pair(ldexpf(v[8 * kb + 2 * e], k), ldexpf(v[8 * kb + 2 * e + 1], k), wh[e], wl[e]);
      h[kb] = op8(wh[0], wh[1], wh[2], wh[3]);
      l[kb] = op8(wl[0], wl[1], wl[2], wl[3]);
    }
  };
  load_q(a.qt + (unit * NR + (Rj < NR ? Rj : 0)) * D, qh, ql, unq);
  if constexpr (KQ) load_q(a.sqt + (unit * NR + (Rj < NR ? Rj : 0)) * D, sh, sl, uns);

  f32x4v oh[8], ol[8], ah[VQ ? 8 : 1], al[VQ ? 8 : 1];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    oh[cb] = ol[cb] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (VQ) ah[cb] = al[cb] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
  }
  float M = -INFINITY, L = 0.0f;                      // row n (replicated over g)

  __syncthreads();                                    // tables
  for (int tbase = t_lo; tbase < tl_b; tbase += TT) {
    const int ntok = min(TT, tl_b - tbase);
    const int nst = (ntok + 15) & ~15;                // whole 16-slot blocks (capacity % 16 == 0)
    const size_t rec0 = unit * a.cap + tbase;
    __syncthreads();                                  // previous tile consumed
    {
      // keys: token tid / 4, coordinates 32 (tid % 4) .. + 31 (and the K spins)
      const int t = tid >> 2, qk = tid & 3;
      const bool ok = t < ntok;
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      if (ok) {
        const uint8_t *r = a.kc + (rec0 + t) * KBYTES;
        if constexpr (KB == 4) {
          const u32x4 x = *(const u32x4 *)(r + 16 * qk);
          w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
        } else if constexpr (KB == 3) {
          const u32x2 x = *(const u32x2 *)(r + 8 * qk);
          w[0] = x.x; w[1] = x.y;
          w[2] = *(const uint32_t *)(r + D / 4 + 4 * qk);
        } else if constexpr (KB == 2) {
          const u32x2 x = *(const u32x2 *)(r + 8 * qk);
          w[0] = x.x; w[1] = x.y;
        } else {
          w[0] = *(const uint32_t *)(r + 4 * qk);
        }
      }
      _Float16 *kd = kt_s + t * KP + 32 * qk;
#pragma unroll
      for (int c8 = 0; c8 < 4; ++c8) {
        f16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = ok ? kc_s[quarter_code<KB>(w, 8 * c8 + e)] : (_Float16)0.0f;
        *(f16x8 *)(kd + 8 * c8) = v;
      }
      if constexpr (KQ) {
        const uint32_t sw = ok ? *(const uint32_t *)(a.ks + (rec0 + t) * (D / 8) + 4 * qk) : 0u;
        _Float16 *pd = kp_s + t * KP + 32 * qk;
#pragma unroll
        for (int by = 0; by < 4; ++by) {
          const u32x2 lo = sp_s[(sw >> (8 * by)) & 15u], hi = sp_s[(sw >> (8 * by + 4)) & 15u];
          *(u32x4 *)(pd + 8 * by) = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
      }
    }
    {
      // values: quad tid / 16 (slots 4 q .. 4 q + 3), piece n (coordinates 8 n .. 8 n + 7)
      const int q = tid >> 4, pc = tid & 15;
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      if (4 * q < nst) {
        const uint8_t *r = a.vc + (rec0 + 4 * q) * VBYTES + 4 * VB * pc;
        if constexpr (VB == 4) {
          const u32x4 x = *(const u32x4 *)r;
          w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
        } else if constexpr (VB == 3) {
          w[0] = *(const uint32_t *)r; w[1] = *(const uint32_t *)(r + 4); w[2] = *(const uint32_t *)(r + 8);
        } else if constexpr (VB == 2) {
          const u32x2 x = *(const u32x2 *)r;
          w[0] = x.x; w[1] = x.y;
        } else {
          w[0] = *(const uint32_t *)r;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        _Float16 o4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          o4[r] = 4 * q + r < ntok ? vc_s[piece_code<VB>(w, j, r)] : (_Float16)0.0f;
        *(u32x2 *)(vt_s + (8 * pc + j) * VP + 4 * q) =
            u32x2{(uint32_t)__builtin_bit_cast(uint16_t, o4[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, o4[1]) << 16),
                  (uint32_t)__builtin_bit_cast(uint16_t, o4[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, o4[3]) << 16)};
      }
    }
    if constexpr (VQ) {
      // value spins: octet tid / 32 (slots 8 o .. 8 o + 7), sketch rows 4 (tid % 32) .. + 3
      const int o = tid >> 5, k0 = 4 * (tid & 31);
      const uint32_t sw = 8 * o < nst ? *(const uint32_t *)(a.vs + (rec0 + 8 * o) * (D / 8) + k0) : 0u;
#pragma unroll
      for (int by = 0; by < 4; ++by) {
        const u32x2 lo = sp_s[(sw >> (8 * by)) & 15u], hi = sp_s[(sw >> (8 * by + 4)) & 15u];
        *(u32x4 *)(st_s + (k0 + by) * VP + 8 * o) = u32x4{lo.x, lo.y, hi.x, hi.y};
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

    // base-2 logits of row n for tokens 16 tb + 4 g + r of block tb
    auto scores = [&](int tb, float (&s)[4]) {
      const _Float16 *kr = kt_s + (16 * tb + n) * KP + 8 * g;
      f32x4v h = {0.0f, 0.0f, 0.0f, 0.0f}, l = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const f16x8 A = *(const f16x8 *)(kr + 32 * kb);
        h = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qh[kb], h, 0, 0, 0);
        l = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, ql[kb], l, 0, 0, 0);
      }
      f32x4v kh = {0.0f, 0.0f, 0.0f, 0.0f}, kl = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (KQ) {
        const _Float16 *pr = kp_s + (16 * tb + n) * KP + 8 * g;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const f16x8 A = *(const f16x8 *)(pr + 32 * kb);
          kh = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, sh[kb], kh, 0, 0, 0);
          kl = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, sl[kb], kl, 0, 0, 0);
        }
      }
      const int t0 = 16 * tb + 4 * g;
      const float4 knv = *(const float4 *)(kn_s + t0);
      const float kn4[4] = {knv.x, knv.y, knv.z, knv.w};
      float kr4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (KQ) {
        const float4 v = *(const float4 *)(kr_s + t0);
        kr4[0] = v.x; kr4[1] = v.y; kr4[2] = v.z; kr4[3] = v.w;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = fmaf(l[r], 1.0f / 2048.0f, h[r]) * unq;
        if constexpr (KQ) v = fmaf(a.kcoef * kr4[r], fmaf(kl[r], 1.0f / 2048.0f, kh[r]) * uns, v);
        v = kn4[r] * v;
        s[r] = (tbase + t0 + r < tl && tbase + t0 + r >= a.t0) ? v : -INFINITY;
      }
    };

    // blocks of this tile that some row of the wave can see, in pairs
    const int nb = tl_w > tbase ? min(TT / 16, (tl_w - tbase + 15) / 16) : 0;
#pragma unroll 1
    for (int tb = 0; tb < nb; tb += 2) {
      float s0[4], s1[4];
      scores(tb, s0);
      if (tb + 1 < nb) {
        scores(tb + 1, s1);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) s1[r] = -INFINITY;
      }
      float s[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[r] = s0[r];
        s[4 + r] = s1[r];
      }
      // ---- online softmax (base 2), row n, 32 tokens ----
      float mloc = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) mloc = fmaxf(mloc, s[e]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      const float Mn = fmaxf(M, mloc);
      const float alpha = (Mn == -INFINITY) ? 1.0f : fast_exp2(M - Mn);
      float p[8], ps = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = (s[e] == -INFINITY) ? 0.0f : fast_exp2(s[e] - Mn);
        ps += p[e];
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      L = fmaf(alpha, L, ps);
      M = Mn;
      // rescale the accumulators (rows 4 g + r) unless no row's max moved
      if (__ballot(alpha != 1.0f)) {
        float al4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) al4[r] = __shfl(alpha, 4 * g + r, 64);
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            oh[cb][r] *= al4[r];
            ol[cb][r] *= al4[r];
            if constexpr (VQ) {
              ah[cb][r] *= al4[r];
              al[cb][r] *= al4[r];
            }
          }
      }
      // ---- A operands: weights of row n for tokens tau(g, e) ----
      uint32_t wch[4], wcl[4], wqh[4] = {0u, 0u, 0u, 0u}, wql[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float c[2], cq[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int e = 2 * e2 + u;
          const int tk = e < 4 ? 16 * tb + 4 * g + e : 16 * (tb + 1) + 4 * g + (e - 4);
          // tokens of zero weight contribute exactly nothing (a stored norm may be +Inf)
          c[u] = p[e] == 0.0f ? 0.0f : p[e] * vn_s[tk];
          cq[u] = VQ ? c[u] * vr_s[tk] : 0.0f;
        }
        split_pair(c[0], c[1], wch[e2], wcl[e2]);
        if constexpr (VQ) split_pair(cq[0], cq[1], wqh[e2], wql[e2]);
      }
      const f16x8 ch = op8(wch[0], wch[1], wch[2], wch[3]), cl = op8(wcl[0], wcl[1], wcl[2], wcl[3]);
      const f16x8 qh8 = op8(wqh[0], wqh[1], wqh[2], wqh[3]), ql8 = op8(wql[0], wql[1], wql[2], wql[3]);
      // ---- O' += P V^, a += (P rho_v) spins: B = column n of coordinate block cb ----
      const int ta = 16 * tb + 4 * g, tb2 = 16 * (tb + 1) + 4 * g;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const _Float16 *vr = vt_s + (16 * cb + n) * VP;
        const u32x2 x0 = *(const u32x2 *)(vr + ta), x1 = *(const u32x2 *)(vr + tb2);
        const f16x8 B = __builtin_bit_cast(f16x8, u32x4{x0.x, x0.y, x1.x, x1.y});
        oh[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ch, B, oh[cb], 0, 0, 0);
        ol[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cl, B, ol[cb], 0, 0, 0);
        if constexpr (VQ) {
          const _Float16 *sr = st_s + (16 * cb + n) * VP;
          const u32x2 y0 = *(const u32x2 *)(sr + ta), y1 = *(const u32x2 *)(sr + tb2);
          const f16x8 Bs = __builtin_bit_cast(f16x8, u32x4{y0.x, y0.y, y1.x, y1.y});
          ah[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh8, Bs, ah[cb], 0, 0, 0);
          al[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql8, Bs, al[cb], 0, 0, 0);
        }
      }
    }
  }
  // partials of rows 4 g + r: M, L, o', a (a split that sees no slot of a
  // row leaves M = -inf, L = 0 and zero sums)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int R = R0 + 4 * g + r;
    const float Mr = __shfl(M, 4 * g + r, 64);
    const float Lr = __shfl(L, 4 * g + r, 64);
    if (R < NR) {
      float *dst = a.part + ((unit * NR + R) * a.splits + split) * (2 + 2 * D);
      if (n == 0) {
        dst[0] = Mr;
        dst[1] = Lr;
      }
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        dst[2 + 16 * cb + n] = fmaf(ol[cb][r], 1.0f / 2048.0f, oh[cb][r]);
        if constexpr (VQ) dst[2 + D + 16 * cb + n] = fmaf(al[cb][r], 1.0f / 2048.0f, ah[cb][r]);
      }
    }
  }
}

}  // namespace kvq
