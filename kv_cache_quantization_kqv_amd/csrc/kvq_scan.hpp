// kvq_scan.hpp -- the decode scan on the matrix cores (head dimension 128).
// Included by kvq_kernels.hpp.
//
// One block (4 waves) per (token split, KV head, group of GT <= 4 query
// heads, batch row), as the merge kernel expects; each wave streams its own
// quarter of the split in blocks of 16 tokens and keeps a running softmax,
// so the main loop has no block barrier.  All three contractions of a token
// block run on v_mfma_f32_16x16x32_f16 (16 x 16 output, 32-deep):
//
//   scores  S[row][t] = sum_k Q[row][k] K^[k][t]     rows 4h + kind, t = token, k = coordinate
//   values  O[c][col] = sum_k V^[c][k] W[k][col]     c = coordinate, k = token of a block pair
//   sketch  A[m][col] = sum_k Sg[m][k] W'[k][col]    m = sketch row, k = token of a block pair
//
// The codebook levels are binary16 values, so the centroid tables are exact
// in one fp16 operand, and sign bits enter as exact fp16 +-1.  The other
// operands carry fp32-level precision as a split x = xh + 2^-11 xl (xh =
// fp16(x), xl = fp16((x - xh) 2^11)): the prepared query and S q' (two rows
// of the A operand), the softmax weights c = w n_v and cq = c rho_v (two
// columns of the B operand).  Two output rows / columns per quantity collect
// sum xh y and sum xl y, combined as hi + lo / 2048.
//
// Lane roles (lane = 16 g + n):
//   scores / softmax : token n of the block, query head g (one pair per lane);
//                      the running max is updated once per pair of blocks;
//                      key operand of step j: coordinates 32 g + 8 j .. + 7
//   value A operand  : coordinate 8 n + j, tokens 4 g .. 4 g + 3 of both blocks
//   sketch A operand : sketch row 8 n + j, tokens of octet g % 2 of block g / 2
//   weight operands  : column 4 h + kind (kind 0/1: value hi/lo, 2/3:
//                      sketch hi/lo) of head h, the lane group's tokens
// The softmax lane layout is turned into the weight-operand layout through a
// small per-wave LDS buffer (one dword per (token, head) and quantity).
//
// Records are read in their stored layout with raw buffer loads (one
// descriptor per array and unit; slots past the scanned range read as zero,
// so the loads need no branch).  Each lane loads exactly the bytes of its
// operand roles: the 16-byte key quarter of its token, and -- the value side
// is stored in token groups (kvq_vgroup.hpp) -- the piece of its quad (token-
// pair or token-quad table indices of its eight coordinates) and the eight
// sketch-row bytes of its token octet, whose bits are the octet's tokens.
// Blocks are aligned to 16 cache slots; slots before the scanned range in the
// first block are masked like those past its end.
#pragma once

namespace kvq {

typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));

// 8 fp16 lanes of an MFMA operand from four dwords.
__device__ __forceinline__ f16x8 op8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(f16x8, u32x4{a, b, c, d});
}

// Delta swap: exchange the bit groups selected by m with those s bits above.
__device__ __forceinline__ uint32_t dswap(uint32_t x, int s, uint32_t m) {
  const uint32_t t = ((x >> s) ^ x) & m;
  return x ^ t ^ (t << s);
}

// Maximum / sum over each row of 16 lanes (DPP), result in every lane of the row.
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}

// Value of lane 4 q + 1 (resp. + 3) in lane 4 q (resp. 4 q + 2): quad_perm [1, 1, 3, 3].
__device__ __forceinline__ float quad_next(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xF5, 0xF, 0xF, false));
}

// fp16 hi/lo split of two non-negative floats: (hi(a), hi(b)) and (lo(a), lo(b)),
// lo = fp16((x - hi) 2^11), packed low half first.  Conversions truncate; the
// remainder captures what the high part drops.
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
  const float ah = (float)__builtin_bit_cast(_Float16, (uint16_t)(hi & 0xFFFFu));
  const float bh = (float)__builtin_bit_cast(_Float16, (uint16_t)(hi >> 16));
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz((a - ah) * 2048.0f, (b - bh) * 2048.0f));
}

// fp16 split of two floats (any sign): words hi and lo (element 0 in the low
// half) with x = h + l 2^-11 to about 2^-22.  h is one rounding of each x, and
// l is taken from exactly that h: the packed word passes through an opaque
// register, so the operand and the remainder cannot come from two separate
// conversions (the compiler may lower one conversion to different
// instructions, whose roundings of a near-tie need not agree).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t &hi, uint32_t &lo) {
  const f32x2 x = {x0, x1};
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
  asm volatile("" : "+v"(hi));
  const f16x2 hv = __builtin_bit_cast(f16x2, hi);
  const f32x2 r = {(x0 - (float)hv[0]) * 2048.0f, (x1 - (float)hv[1]) * 2048.0f};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, f16x2));
}

template <int KB, bool KQ, int VB, bool VQ>
struct ScanShape {
  static constexpr int D = 128;
  static constexpr int KREC = D * KB / 8, VREC = D * VB / 8, SREC = D / 8;
  // key operand table: byte (KB 4) or 6-bit index (KB 3) of two codes -> 4
  // bytes; byte (KB 2) or nibble (KB 1) of four codes -> 8 bytes
  static constexpr bool KPAIR = KB >= 3;
  static constexpr int KENT = KB == 4 ? 256 : KB == 3 ? 64 : KB == 2 ? 256 : 16;
  static constexpr int KTB = KENT * (KPAIR ? 4 : 8);
  static constexpr int KW = KB == 4 ? 4 : KB == 3 ? 3 : KB == 2 ? 2 : 1;   // key dwords per lane
  // value operand table: token-pair index (VB 4: a byte, VB 3: 6 bits) -> 4
  // bytes, or token-quad index (VB 2: byte, VB 1: nibble) -> 8 bytes.  (Small
  // tables matter: random reads of a 64-entry table meet fewer LDS bank
  // conflicts than those of a 256-entry one.)
  static constexpr bool VQUAD = VB <= 2;
  static constexpr int VENT = VB == 1 ? 16 : VB == 3 ? 64 : 256;
  static constexpr int VTB = VENT * (VQUAD ? 8 : 4);
  static constexpr int PB = 4 * VB;                                         // value piece bytes per lane
  static constexpr bool SPIN = KQ || VQ;
  static constexpr int NS = 2 + 2 * D;                                      // partial floats per head
};

// One token block's raw data in registers.  Keys and norms are loaded per
// scored token; the value piece is the lane's (quad g of the block,
// coordinates 8n .. 8n+7); the value sign bytes (rows 8n .. 8n+7 of octet
// g % 2) are loaded by the lanes g / 2 == block parity within the pair.
template <int KB, bool KQ, int VB, bool VQ>
struct ScanBlock {
  using SS = ScanShape<KB, KQ, VB, VQ>;
  uint32_t k[SS::KW];    // key bytes of token n for coordinates 32 g .. 32 g + 31
  uint32_t ks;           // key sign bytes 4 g .. 4 g + 3 of token n (rows 32 g .. 32 g + 31)
  uint32_t nk, rk, nv, rv;   // fp16 bits of the key norm, key residual norm, value norm, value residual norm
  uint32_t v[VB];        // value piece
  u32x2 sg;              // value sign bytes (zero in lanes of the other parity)
};

// Buffer descriptors of one (batch row, KV head) unit: each covers the unit's
// slots [0, t0 + n_ctx) of one array, so a load past the scanned range reads
// zero (hardware range check) and needs no branch.
struct ScanRsrc {
  __amdgpu_buffer_rsrc_t kc, ks, vc, vs, kn, kr, vn, vr;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t unit_rsrc(const void *base, size_t unit_off,
                                                           uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)((const uint8_t *)base + unit_off), (short)0,
                                           (int)bytes, 0x00020000);
}

// Loads of the scan stream data that is read once per step: non-temporal
// (cache-policy bit 1), so it does not evict what stays resident.
template <int KB, bool KQ, int VB, bool VQ>
__device__ __forceinline__ void scan_load(ScanBlock<KB, KQ, VB, VQ> &R, const ScanRsrc &rs, int slot0,
                                          int tb, int n, int g, int par) {
  using SS = ScanShape<KB, KQ, VB, VQ>;
  constexpr int NT = 2;
  const uint32_t tk = (uint32_t)(slot0 + tb + n);       // slot of this lane's scored token
  const uint32_t ko = tk * SS::KREC;
  if constexpr (KB == 4) {
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rs.kc, ko + 16 * g, 0, NT);
    R.k[0] = w.x; R.k[1] = w.y; R.k[2] = w.z; R.k[3] = w.w;
  } else if constexpr (KB == 3) {
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rs.kc, ko + 8 * g, 0, NT);
    R.k[0] = w.x; R.k[1] = w.y;
    R.k[2] = __builtin_amdgcn_raw_buffer_load_b32(rs.kc, ko + SS::D / 4 + 4 * g, 0, NT);
  } else if constexpr (KB == 2) {
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rs.kc, ko + 8 * g, 0, NT);
    R.k[0] = w.x; R.k[1] = w.y;
  } else {
    R.k[0] = __builtin_amdgcn_raw_buffer_load_b32(rs.kc, ko + 4 * g, 0, NT);
  }
  R.ks = KQ ? __builtin_amdgcn_raw_buffer_load_b32(rs.ks, tk * SS::SREC + 4 * g, 0, NT) : 0u;
  R.nk = __builtin_amdgcn_raw_buffer_load_b16(rs.kn, 2 * tk, 0, NT);
  R.rk = KQ ? __builtin_amdgcn_raw_buffer_load_b16(rs.kr, 2 * tk, 0, NT) : 0u;
  R.nv = __builtin_amdgcn_raw_buffer_load_b16(rs.vn, 2 * tk, 0, NT);
  R.rv = VQ ? __builtin_amdgcn_raw_buffer_load_b16(rs.vr, 2 * tk, 0, NT) : 0u;
  const int lane = 16 * g + n;
  const uint32_t t16 = (uint32_t)(slot0 + tb);          // a multiple of 16
  const uint32_t vo = t16 * SS::VREC + (uint32_t)(SS::PB * lane);
  if constexpr (VB == 4) {
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rs.vc, vo, 0, NT);
    R.v[0] = w.x; R.v[1] = w.y; R.v[2] = w.z; R.v[3] = w.w;
  } else if constexpr (VB == 3) {
    const u32x3 w = __builtin_amdgcn_raw_buffer_load_b96(rs.vc, vo, 0, NT);
    R.v[0] = w.x; R.v[1] = w.y; R.v[2] = w.z;
  } else if constexpr (VB == 2) {
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rs.vc, vo, 0, NT);
    R.v[0] = w.x; R.v[1] = w.y;
  } else {
    R.v[0] = __builtin_amdgcn_raw_buffer_load_b32(rs.vc, vo, 0, NT);
  }
  R.sg = u32x2{0u, 0u};
  if constexpr (VQ) {
    // lanes of the other parity read at an offset past every range (zero)
    const uint32_t so = (g >> 1) == par ? t16 * SS::SREC + 128u * (uint32_t)(g & 1) + 8u * (uint32_t)n
                                        : 0xFFFFFFF0u;
    R.sg = __builtin_amdgcn_raw_buffer_load_b64(rs.vs, so, 0, NT);
  }
}

// B operand of the score product for step j: key centroids of coordinates
// 32 g + 8 j .. + 7 of token n (fp16, coordinate order).
template <int KB>
__device__ __forceinline__ f16x8 key_operand(const uint32_t *k, int j, const uint8_t *tab) {
  if constexpr (KB == 4) {
    const uint32_t w = k[j];
    const uint32_t t0 = *(const uint32_t *)(tab + 4 * (w & 255u));
    const uint32_t t1 = *(const uint32_t *)(tab + 4 * ((w >> 8) & 255u));
    const uint32_t t2 = *(const uint32_t *)(tab + 4 * ((w >> 16) & 255u));
    const uint32_t t3 = *(const uint32_t *)(tab + 4 * (w >> 24));
    return op8(t0, t1, t2, t3);
  } else if constexpr (KB == 3) {
    // 2-bit plane: 16 bits of coordinates 8 j .. 8 j + 7; 1-bit plane: byte j
    const uint32_t lo = (k[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    const uint32_t hb = (k[2] >> (8 * j)) & 255u;
    uint32_t t[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t idx = ((lo >> (4 * b)) & 15u) | (((hb >> (2 * b)) & 3u) << 4);
      t[b] = *(const uint32_t *)(tab + 4 * idx);
    }
    return op8(t[0], t[1], t[2], t[3]);
  } else if constexpr (KB == 2) {
    const uint32_t w = (k[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    const u32x2 t0 = *(const u32x2 *)(tab + 8 * (w & 255u));
    const u32x2 t1 = *(const u32x2 *)(tab + 8 * (w >> 8));
    return op8(t0.x, t0.y, t1.x, t1.y);
  } else {
    const uint32_t by = (k[0] >> (8 * j)) & 255u;
    const u32x2 t0 = *(const u32x2 *)(tab + 8 * (by & 15u));
    const u32x2 t1 = *(const u32x2 *)(tab + 8 * (by >> 4));
    return op8(t0.x, t0.y, t1.x, t1.y);
  }
}

// A operand of value step j (coordinate 8n + j) over a block pair: slots
// 0..3 = tokens 4g .. 4g+3 of the first block (piece a), 4..7 = those of the
// second (piece b).  value_field: the byte offset of field u's entry in the
// 4-byte pair table.  Width 3 stores fields 0..11 as 4 P in their bytes (one
// mask), and h3a / h3b gather fields 12..15 of a piece, also as 4 P, into the
// bytes of one dword (once per block).
template <int VB>
__device__ __forceinline__ uint32_t value_field(const uint32_t *v, uint32_t h3, int u) {
  if constexpr (VB == 4) return 4 * ((v[u >> 2] >> (8 * (u & 3))) & 255u);
  if (u < 12) return (v[u >> 2] >> (8 * (u & 3))) & 0xFCu;
  return (h3 >> (8 * (u - 12))) & 255u;
}

template <int VB>
__device__ __forceinline__ f16x8 value_operand(const uint32_t *va, uint32_t h3a, const uint32_t *vb,
                                               uint32_t h3b, int j, const uint8_t *tab) {
  if constexpr (VB == 4 || VB == 3) {
    const uint32_t t0 = *(const uint32_t *)(tab + value_field<VB>(va, h3a, 2 * j));
    const uint32_t t1 = *(const uint32_t *)(tab + value_field<VB>(va, h3a, 2 * j + 1));
    const uint32_t t2 = *(const uint32_t *)(tab + value_field<VB>(vb, h3b, 2 * j));
    const uint32_t t3 = *(const uint32_t *)(tab + value_field<VB>(vb, h3b, 2 * j + 1));
    return op8(t0, t1, t2, t3);
  } else if constexpr (VB == 2) {
    const u32x2 ta = *(const u32x2 *)(tab + 8 * ((va[j >> 2] >> (8 * (j & 3))) & 255u));
    const u32x2 tb = *(const u32x2 *)(tab + 8 * ((vb[j >> 2] >> (8 * (j & 3))) & 255u));
    return op8(ta.x, ta.y, tb.x, tb.y);
  } else {
    const u32x2 ta = *(const u32x2 *)(tab + 8 * ((va[0] >> (4 * j)) & 15u));
    const u32x2 tb = *(const u32x2 *)(tab + 8 * ((vb[0] >> (4 * j)) & 15u));
    return op8(ta.x, ta.y, tb.x, tb.y);
  }
}

template <int KB, bool KQ, int VB, bool VQ>
__global__ __launch_bounds__(256) void scan_kernel(const DecodeArgs a) {
  using SS = ScanShape<KB, KQ, VB, VQ>;
  using SB = ScanBlock<KB, KQ, VB, VQ>;
  constexpr int D = SS::D, NS = SS::NS;
  __shared__ __attribute__((aligned(16))) uint8_t kt_s[SS::KTB];
  __shared__ __attribute__((aligned(16))) uint8_t vt_s[SS::VTB];
  // nibble -> 4 fp16 spins (+1 where the bit is set, else -1), element e = bit e
  __shared__ __attribute__((aligned(16))) u32x2 sp_s[SS::SPIN ? 16 : 1];
  // per wave: X = (ch, cl) and Z = (cqh, cql) of [block parity][head][token]
  __shared__ __attribute__((aligned(16))) uint32_t wx_s[4][2][4][16];
  __shared__ __attribute__((aligned(16))) uint32_t wz_s[4][2][4][16];
  __shared__ __attribute__((aligned(16))) float ep_s[4][4][NS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: a scalar loop below
  const int n = lane & 15, g = lane >> 4;
  const int GT = a.Gtot < 4 ? a.Gtot : 4;
  const int split = blockIdx.x;
  const int hkv = blockIdx.y / a.HG, hgrp = blockIdx.y - (blockIdx.y / a.HG) * a.HG;
  const int b = blockIdx.z;
  const int hq0 = hkv * a.Gtot + hgrp * GT;
  const size_t unit = (size_t)b * a.Hkv + hkv;
  const size_t unitg = unit * a.HG + hgrp;
  // per-unit buffer descriptors over slots [0, t0 + n_ctx)
  // scanned slots [t0, t0 + n_ctx) in blocks aligned to 16 slots from A; the
  // descriptors reach the end of the last block (capacity is a multiple of 16)
  const int A = a.t0 & ~15, lead = a.t0 - A, span = lead + a.n_ctx;
  const uint32_t nslot = (uint32_t)((a.t0 + a.n_ctx + 15) & ~15);
  const size_t us = unit * (size_t)a.cap;
  ScanRsrc rs;
  rs.kc = unit_rsrc(a.kc, us * SS::KREC, nslot * SS::KREC);
  rs.vc = unit_rsrc(a.vc, us * SS::VREC, nslot * SS::VREC);
  rs.kn = unit_rsrc(a.kn, us * 2, nslot * 2);
  rs.vn = unit_rsrc(a.vn, us * 2, nslot * 2);
  rs.ks = rs.kr = rs.vs = rs.vr = rs.kc;
  if constexpr (KQ) {
    rs.ks = unit_rsrc(a.ks, us * SS::SREC, nslot * SS::SREC);
    rs.kr = unit_rsrc(a.kr, us * 2, nslot * 2);
  }
  if constexpr (VQ) {
    rs.vs = unit_rsrc(a.vs, us * SS::SREC, nslot * SS::SREC);
    rs.vr = unit_rsrc(a.vr, us * 2, nslot * 2);
  }

  // ---- tables (shared by the block): fp16 levels (exact) in index order ----
  auto h16 = [](float c) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)c); };
  for (int p = tid; p < SS::KENT; p += 256) {
    if constexpr (SS::KPAIR) {
      int ca, cb;
      pair_codes<KB>(p, ca, cb);
      *(uint32_t *)(kt_s + 4 * p) = h16(a.kcent[ca]) | (h16(a.kcent[cb]) << 16);
    } else {
      constexpr int M = (1 << KB) - 1;
      *(u32x2 *)(kt_s + 8 * p) = u32x2{h16(a.kcent[p & M]) | (h16(a.kcent[(p >> KB) & M]) << 16),
                                       h16(a.kcent[(p >> (2 * KB)) & M]) |
                                           (h16(a.kcent[(p >> (3 * KB)) & M]) << 16)};
    }
  }
  // value table: the tokens of a pair / quad index (fields as in the
  // token-group storage), in token order
  for (int p = tid; p < SS::VENT; p += 256) {
    constexpr int FW = VB == 3 ? 3 : VB, M = (1 << VB) - 1;
    auto c = [&](int r) { return h16(a.vcent[(p >> (FW * r)) & M]); };
    if constexpr (SS::VQUAD) *(u32x2 *)(vt_s + 8 * p) = u32x2{c(0) | (c(1) << 16), c(2) | (c(3) << 16)};
    else *(uint32_t *)(vt_s + 4 * p) = c(0) | (c(1) << 16);
  }
  if constexpr (SS::SPIN) {
    if (tid < 16) {
      uint32_t w[2];
#pragma unroll
      for (int q = 0; q < 2; ++q)
        w[q] = (((tid >> (2 * q)) & 1) ? 0x3C00u : 0xBC00u) | ((((tid >> (2 * q + 1)) & 1) ? 0x3C00u : 0xBC00u) << 16);
      sp_s[tid] = u32x2{w[0], w[1]};
    }
  }
  // the 8 spins of a sign byte (element e = bit e)
  auto spins = [&](uint32_t x) {
    const u32x2 lo = sp_s[x & 15u], hi = sp_s[(x >> 4) & 15u];
    return op8(lo.x, lo.y, hi.x, hi.y);
  };

  // ---- q' = R q qscale of the block's heads, when not prepared beforehand ------
  // wave h takes head h: lane l holds coordinates l and l + 64, the butterfly
  // stages run in ascending h as in the query-preparation kernel (partner
  // lane l ^ h; the last stage within the lane), with the same operations, so
  // q' is bit for bit the one that kernel writes
  __shared__ __attribute__((aligned(16))) float qv_s[4 * D];
  if (a.qsrc) {
    if (wave < GT) {
      const size_t row = (size_t)b * a.Hq + hq0 + wave;
      float x0, x1;
      if (a.q_bf16) {
        x0 = bf16_to_f32(((const uint16_t *)a.qsrc)[row * D + lane]);
        x1 = bf16_to_f32(((const uint16_t *)a.qsrc)[row * D + lane + 64]);
      } else {
        x0 = ((const float *)a.qsrc)[row * D + lane];
        x1 = ((const float *)a.qsrc)[row * D + lane + 64];
      }
      if (a.rk == RK_RHT) {
        if ((a.rsign[lane >> 5] >> (lane & 31)) & 1u) x0 = -x0;
        if ((a.rsign[2 + (lane >> 5)] >> (lane & 31)) & 1u) x1 = -x1;
      }
      if (a.rk == RK_WHT || a.rk == RK_RHT) {
#pragma unroll
        for (int h = 1; h < 64; h <<= 1) {
          const float q0 = __shfl_xor(x0, h, 64), q1 = __shfl_xor(x1, h, 64);
          x0 = (lane & h) ? (q0 - x0) : (x0 + q0);
          x1 = (lane & h) ? (q1 - x1) : (x1 + q1);
        }
        const float lo = x0, hi = x1;
        x0 = lo + hi;
        x1 = lo - hi;
      }
      qv_s[lane * GT + wave] = x0 * a.qscale;
      qv_s[(lane + 64) * GT + wave] = x1 * a.qscale;
    }
    __syncthreads();
  }

  // ---- prepared query as the A operand of the score product -------------------
  // lane (row = 4 h + kind, g); step j slot e <-> coordinate 32 g + 8 j + e;
  // kind 0: q' hi, kind 1: q' lo (kinds 2, 3: zero here)
  const int qrow = n, qh_ = qrow >> 2, qkind = qrow & 3;
  f16x8 qa[4];
  float unsc_q;
  {
    const float *qv = a.qsrc ? qv_s : a.qt + unitg * D * GT;
    float v[32];
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      v[c] = qh_ < GT ? qv[(32 * g + c) * GT + qh_] : 0.0f;
      m = fmaxf(m, fabsf(v[c]));
    }
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    int ex = 0;
    const bool fin = m > 0.0f && m <= 3.0e38f;
    if (fin) (void)frexpf(m, &ex);
    const int k = fin ? 14 - ex : 0;
    unsc_q = ldexpf(1.0f, -k);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t hi, lo;
        split_pair(ldexpf(v[8 * j + 2 * e], k), ldexpf(v[8 * j + 2 * e + 1], k), hi, lo);
        w[e] = qkind == 0 ? hi : (qkind == 1 ? lo : 0u);
      }
      qa[j] = op8(w[0], w[1], w[2], w[3]);
    }
  }
  // K sketch (QKQV): rows 4 h + 2 / 4 h + 3 carry S q' hi / lo, slot e of step
  // j <-> sketch row 32 g + 8 j + e
  f16x8 qs[KQ ? 4 : 1];
  float unsc_s = 0.0f;
  if constexpr (KQ) {
    const float *sv = a.sqt + unitg * D * GT;
    float v[32];
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      v[c] = qh_ < GT ? sv[(32 * g + c) * GT + qh_] : 0.0f;
      m = fmaxf(m, fabsf(v[c]));
    }
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    int ex = 0;
    const bool fin = m > 0.0f && m <= 3.0e38f;
    if (fin) (void)frexpf(m, &ex);
    const int k = fin ? 14 - ex : 0;
    unsc_s = ldexpf(1.0f, -k);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t hi, lo;
        split_pair(ldexpf(v[8 * j + 2 * e], k), ldexpf(v[8 * j + 2 * e + 1], k), hi, lo);
        w[e] = qkind == 2 ? hi : (qkind == 3 ? lo : 0u);
      }
      qs[j] = op8(w[0], w[1], w[2], w[3]);
    }
  }
  // scale factors of the softmax lane's head g (row 4 g of the operand lanes)
  const float unscale = __shfl(unsc_q, 4 * g, 64);
  const float unscale_s = KQ ? __shfl(unsc_s, 4 * g, 64) : 0.0f;
  const bool head_ok = g < GT;

  // weight-operand lane role: column 4 hc + kind
  const int hc = n >> 2, wkind = n & 3;
  const uint32_t selV = wkind == 0 ? 0x05040100u : (wkind == 1 ? 0x07060302u : 0x0C0C0C0Cu);
  const uint32_t selS = wkind == 2 ? 0x05040100u : (wkind == 3 ? 0x07060302u : 0x0C0C0C0Cu);

  // ---- this wave's tokens ----------------------------------------------------
  // The unit's aligned range is cut into 64-token chunks; its W = 4 splits
  // workers take chunks worker, worker + W, ... (interleaved), so the waves
  // resident at one time read neighbouring memory of each array (a sweep, not
  // W separate streams).  Token order does not matter to the online softmax.
  const int W = 4 * a.splits;
  const int worker = 4 * split + wave;
  const int nchunk = (span + 63) >> 6;

  f32x4v acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
  float M = -3.0e38f, L = 0.0f;
  __syncthreads();   // tables

  uint32_t(*wx)[4][16] = wx_s[wave];
  uint32_t(*wz)[4][16] = wz_s[wave];
  const uint8_t *vtab = (const uint8_t *)vt_s;

  // base-2 logit of (token n, head g) of one block, -inf past the range
  auto score = [&](const SB &R, int tb) {
    // two independent accumulation chains (a chain waits for each result)
    f32x4v sc0 = {0.0f, 0.0f, 0.0f, 0.0f}, sc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      sc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[j], key_operand<KB>(R.k, j, kt_s), sc0, 0, 0, 0);
      sc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[j + 1], key_operand<KB>(R.k, j + 1, kt_s), sc1, 0, 0, 0);
    }
    if constexpr (KQ) {
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        const f16x8 sg0 = spins(R.ks >> (8 * j));
        const f16x8 sg1 = spins(R.ks >> (8 * j + 8));
        sc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qs[j], sg0, sc0, 0, 0, 0);
        sc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qs[j + 1], sg1, sc1, 0, 0, 0);
      }
    }
    const f32x4v sc = sc0 + sc1;
    float s = fmaf(sc[1], 1.0f / 2048.0f, sc[0]) * unscale;
    if constexpr (KQ) {
      const float sk = fmaf(sc[3], 1.0f / 2048.0f, sc[2]) * unscale_s;
      s = fmaf(a.kcoef * f16_bits_to_f32((uint16_t)R.rk), sk, s);
    }
    s *= f16_bits_to_f32((uint16_t)R.nk);
    return (head_ok && tb + n >= lead && tb + n < span) ? s : -INFINITY;
  };
  // weights of one block into the exchange buffers of parity par
  auto weights = [&](const SB &R, float s, int par) {
    const float w = fast_exp2(s - M);
    L += w;
    // masked tokens contribute exactly nothing (their stored norm may be +Inf)
    const float c = s == -INFINITY ? 0.0f : w * f16_bits_to_f32((uint16_t)R.nv);
    const float cq = VQ ? c * f16_bits_to_f32((uint16_t)R.rv) : 0.0f;
    uint32_t hi, lo;
    split2(c, cq, hi, lo);
    wx[par][g][n] = __builtin_amdgcn_perm(lo, hi, 0x05040100u);   // (ch, cl)
    if constexpr (VQ) wz[par][g][n] = __builtin_amdgcn_perm(lo, hi, 0x07060302u);   // (cqh, cql)
  };
  // value product of a block pair: A = centroids of the lanes' pieces, B =
  // weights hi (kind 0) / lo (kind 1) of head hc for the same tokens
  auto values = [&](const SB &RA, const SB &RB) {
    const u32x4 XA = *(const u32x4 *)&wx[0][hc][4 * g];
    const u32x4 XB = *(const u32x4 *)&wx[1][hc][4 * g];
    const f16x8 bv = op8(__builtin_amdgcn_perm(XA.y, XA.x, selV), __builtin_amdgcn_perm(XA.w, XA.z, selV),
                         __builtin_amdgcn_perm(XB.y, XB.x, selV), __builtin_amdgcn_perm(XB.w, XB.z, selV));
    uint32_t h3a = 0u, h3b = 0u;
    if constexpr (VB == 3) {
      h3a = ((RA.v[0] & 0x03030303u) << 2) | ((RA.v[1] & 0x03030303u) << 4) | ((RA.v[2] & 0x03030303u) << 6);
      h3b = ((RB.v[0] & 0x03030303u) << 2) | ((RB.v[1] & 0x03030303u) << 4) | ((RB.v[2] & 0x03030303u) << 6);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(value_operand<VB>(RA.v, h3a, RB.v, h3b, j, vtab),
                                                      bv, acc[j], 0, 0, 0);
  };
  // sketch product of a block pair: lane group g covers octet g % 2 of block
  // g / 2 (slot e <-> token 8 (g % 2) + e of that block); A = spins of the
  // lane's sign byte j (row 8 n + j, bit e = token e)
  auto sketch = [&](u32x2 sg) {
    const uint32_t(*zq)[16] = wz[g >> 1];
    const u32x4 Z0 = *(const u32x4 *)&zq[hc][8 * (g & 1)];
    const u32x4 Z1 = *(const u32x4 *)&zq[hc][8 * (g & 1) + 4];
    const f16x8 bz = op8(__builtin_amdgcn_perm(Z0.y, Z0.x, selS), __builtin_amdgcn_perm(Z0.w, Z0.z, selS),
                         __builtin_amdgcn_perm(Z1.y, Z1.x, selS), __builtin_amdgcn_perm(Z1.w, Z1.z, selS));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t x = ((j < 4 ? sg.x : sg.y) >> (8 * (j & 3))) & 255u;
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(spins(x), bz, acc[j], 0, 0, 0);
    }
  };
  // a pair of token blocks: scores of both, one running-max update, then the
  // weighted value and sketch products with the same reference max
  auto process_pair = [&](const SB &RA, const SB &RB, int tb) {
    const float sA = score(RA, tb);
    const float sB = score(RB, tb + 16);
    const float bm = row_max16(fmaxf(sA, sB));
    if (__ballot(bm > M)) {
      const float Mn = fmaxf(M, bm);
      const float al = fast_exp2(M - Mn);
      L *= al;
      M = Mn;
      const float alc = __shfl(al, 16 * hc, 64);   // alpha of the accumulator lane's head
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= alc;
    }
    weights(RA, sA, 0);
    weights(RB, sB, 1);
    wave_sync();
    values(RA, RB);
    if constexpr (VQ) sketch(RA.sg | RB.sg);
    wave_sync();   // the exchange buffers are rewritten by the next pair
  };

  // ---- main loop: a pair of blocks per step, two pairs in flight ------------
  SB R0, R1, R2, R3;
  const int s0 = A;
  // issued in block order (the loop head's wait counts assume it)
  const int tfirst = 64 * min(worker, nchunk);
  __builtin_amdgcn_sched_barrier(0);
  scan_load(R0, rs, s0, tfirst, n, g, 0);
  scan_load(R1, rs, s0, tfirst + 16, n, g, 1);
  __builtin_amdgcn_sched_barrier(0);
  scan_load(R2, rs, s0, tfirst + 32, n, g, 0);
  scan_load(R3, rs, s0, tfirst + 48, n, g, 1);
  __builtin_amdgcn_sched_barrier(0);
  // (the scheduling barriers keep each refill between the two pair steps, so
  // a pair's data is requested a full pair step before it is used)
  for (int ci = worker; ci < nchunk; ci += W) {
    const int tb = 64 * ci;
    const int tn = 64 * min(ci + W, nchunk);   // next chunk (past the end: zeros, unused)
    process_pair(R0, R1, tb);
    __builtin_amdgcn_sched_barrier(0);
    scan_load(R0, rs, s0, tn, n, g, 0);
    scan_load(R1, rs, s0, tn + 16, n, g, 1);
    __builtin_amdgcn_sched_barrier(0);
    process_pair(R2, R3, tb + 32);
    __builtin_amdgcn_sched_barrier(0);
    scan_load(R2, rs, s0, tn + 32, n, g, 0);
    scan_load(R3, rs, s0, tn + 48, n, g, 1);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- epilogue: per-wave partials through LDS, then the block's partial ----
  {
    float l = L;
    l += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(l), 0xB1, 0xF, 0xF, false));
    l += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(l), 0x4E, 0xF, 0xF, false));
    l += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(l), 0x141, 0xF, 0xF, false));
    l += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(l), 0x140, 0xF, 0xF, false));
    if (n == 0) {
      ep_s[wave][g][0] = M;
      ep_s[wave][g][1] = l;
    }
  }
  // lanes of kind 0 (values) and 2 (sketch) combine hi + lo / 2048 of their pair
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = fmaf(quad_next(acc[j][r]), 1.0f / 2048.0f, acc[j][r]);
      const int coord = 32 * g + 8 * r + j;
      if (wkind == 0) ep_s[wave][hc][2 + coord] = v;
      else if (wkind == 2 && VQ) ep_s[wave][hc][2 + D + coord] = v;
    }
  __syncthreads();
  for (int idx = tid; idx < 4 * NS; idx += 256) {
    const int h = idx / NS, kk = idx - h * NS;
    if (h >= GT) continue;
    float mw[4], mx = -3.0e38f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mw[w] = ep_s[w][h][0];
      mx = fmaxf(mx, mw[w]);
    }
    float v;
    if (kk == 0) {
      v = mx > -3.0e38f ? mx : -INFINITY;
    } else if (!VQ && kk >= 2 + D) {
      v = 0.0f;
    } else {
      v = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) v = fmaf(fast_exp2(mw[w] - mx), ep_s[w][h][kk], v);
    }
    a.part[(((size_t)b * a.Hq + hq0 + h) * a.splits + split) * NS + kk] = v;
  }
}

}  // namespace kvq
