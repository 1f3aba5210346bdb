// kvq_vgroup.hpp -- token-group storage of the value side at head dimension
// 128.  Included by kvq_kernels.hpp.
//
// The pages fix no storage format.  This library stores the value codes of
// four neighbouring slots, and the value sign bits of eight, in shared bytes
// laid out in the order the decode scan's matrix operands consume them, so
// the scan reads ready-made table indices instead of re-packing bits of
// separate records (the transposition is paid once, when a token is written):
//
//   codes (width b, R = 16 b bytes per slot): slots 4q .. 4q+3 own bytes
//   [4q R, 4q R + 4R).  Piece n (coordinates 8n .. 8n+7) sits at 4 b n.  With
//   c_r(j) = code of slot 4q + r at coordinate 8n + j:
//     b 4: byte 2j + p = c_{2p}(j) | c_{2p+1}(j) << 4                  (pair index)
//     b 3: field u = 2j + p holds P = c_{2p}(j) | c_{2p+1}(j) << 3; fields
//          0..11 are bits 2..7 of bytes 0..11 (a byte with its low two bits
//          cleared is 4 P, the byte offset of entry P in a 4-byte table),
//          field 12 + m has its bit pairs (0,1), (2,3), (4,5) in bits 0, 1
//          of bytes m, 4 + m, 8 + m
//     b 2: byte j = c_0(j) | c_1(j) << 2 | c_2(j) << 4 | c_3(j) << 6   (quad index)
//     b 1: bits 4j .. 4j+3 = c_0(j) | c_1(j) << 1 | c_2(j) << 2 | c_3(j) << 3
//   sign bits: slots 8o .. 8o+7 own bytes [128 o, 128 o + 128); bit e of
//   byte 128 o + k is the sign of slot 8o + e at sketch row k.
//
// A group never straddles two (batch row, KV head) units: caches with this
// layout have a capacity that is a multiple of 16.
#pragma once

namespace kvq {

// ---- readers (slot numbers count from the array base; units start at
// multiples of 16 slots, so local and global group boundaries agree) ---------

template <int VB>
__device__ __forceinline__ uint32_t vg_code(const uint8_t *vc, size_t slot, int c) {
  const uint8_t *piece = vc + (slot >> 2) * (64 * VB) + (size_t)(c >> 3) * (4 * VB);
  const int r = (int)(slot & 3), j = c & 7;
  if constexpr (VB == 4) {
    return (piece[2 * j + (r >> 1)] >> (4 * (r & 1))) & 15u;
  } else if constexpr (VB == 3) {
    const int u = 2 * j + (r >> 1);
    uint32_t P;
    if (u < 12) {
      P = piece[u] >> 2;
    } else {
      const int m = u - 12;
      P = (piece[m] & 3u) | ((piece[4 + m] & 3u) << 2) | ((piece[8 + m] & 3u) << 4);
    }
    return (P >> (3 * (r & 1))) & 7u;
  } else if constexpr (VB == 2) {
    return (piece[j] >> (2 * r)) & 3u;
  } else {
    return (piece[j >> 1] >> (4 * (j & 1) + r)) & 1u;
  }
}

__device__ __forceinline__ uint32_t vg_sign(const uint8_t *vs, size_t slot, int k) {
  return (vs[(slot >> 3) * 128 + (size_t)k] >> (slot & 7)) & 1u;
}

// ---- encoders ----------------------------------------------------------------

// Delta swap: exchange the bit groups selected by m with those s bits above.
__device__ __forceinline__ uint32_t vg_dswap(uint32_t x, int s, uint32_t m) {
  const uint32_t t = ((x >> s) ^ x) & m;
  return x ^ t ^ (t << s);
}

// Bytes j of (x, y) interleaved: byte j of the result = nibble j of x | nibble
// j of y << 4, for j = 4h .. 4h + 3 (h = 0 or 1).
__device__ __forceinline__ uint32_t vg_nib_pairs(uint32_t x, uint32_t y, int h) {
  return vg_dswap(__builtin_amdgcn_perm(y, x, h ? 0x07030602u : 0x05010400u), 4, 0x00F000F0u);
}

// One piece from the nibble codes of the quad's four slots: N[r] = nibble
// codes of coordinates 8n .. 8n+7 of slot r (coordinate 8n + j in nibble j,
// bits above the width zero).  w: the piece's VB dwords.
template <int VB>
__device__ __forceinline__ void vg_piece(const uint32_t (&N)[4], uint32_t (&w)[VB]) {
  if constexpr (VB == 4) {
    const uint32_t a0 = vg_nib_pairs(N[0], N[1], 0), a1 = vg_nib_pairs(N[0], N[1], 1);
    const uint32_t b0 = vg_nib_pairs(N[2], N[3], 0), b1 = vg_nib_pairs(N[2], N[3], 1);
    w[0] = __builtin_amdgcn_perm(b0, a0, 0x05010400u);
    w[1] = __builtin_amdgcn_perm(b0, a0, 0x07030602u);
    w[2] = __builtin_amdgcn_perm(b1, a1, 0x05010400u);
    w[3] = __builtin_amdgcn_perm(b1, a1, 0x07030602u);
  } else if constexpr (VB == 3) {
    // byte j of q_p(h) = P(j, p) (second code moved from bit 4 to bit 3)
    uint32_t q[2][2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t y = vg_nib_pairs(N[2 * p], N[2 * p + 1], h);
        q[p][h] = (y & 0x0F0F0F0Fu) | ((y >> 1) & 0x78787878u);
      }
    // fields 0..11 move to bits 2..7 of their bytes (6-bit values: nothing
    // crosses a byte), fields 12..15 fill bits 0, 1
    const uint32_t t = __builtin_amdgcn_perm(q[1][1], q[0][1], 0x07030602u);   // 12..15
    w[0] = (__builtin_amdgcn_perm(q[1][0], q[0][0], 0x05010400u) << 2) | (t & 0x03030303u);
    w[1] = (__builtin_amdgcn_perm(q[1][0], q[0][0], 0x07030602u) << 2) | ((t >> 2) & 0x03030303u);
    w[2] = (__builtin_amdgcn_perm(q[1][1], q[0][1], 0x05010400u) << 2) | ((t >> 4) & 0x03030303u);
  } else if constexpr (VB == 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t a = vg_nib_pairs(N[0], N[1], h), b = vg_nib_pairs(N[2], N[3], h);
      a = (a & 0x03030303u) | ((a >> 2) & 0x0C0C0C0Cu);
      b = (b & 0x03030303u) | ((b >> 2) & 0x0C0C0C0Cu);
      w[h] = a | (b << 4);
    }
  } else {
    w[0] = N[0] | (N[1] << 1) | (N[2] << 2) | (N[3] << 3);
  }
}

// 8 x 8 bit transpose: byte e of (lo, hi) (e = 0..3 in lo, 4..7 in hi) is row
// e; afterwards byte j holds bit j of every row (bit e = row e).
__device__ __forceinline__ void vg_transpose8(uint32_t &lo, uint32_t &hi) {
  lo = vg_dswap(vg_dswap(lo, 7, 0x00AA00AAu), 14, 0x0000CCCCu);
  hi = vg_dswap(vg_dswap(hi, 7, 0x00AA00AAu), 14, 0x0000CCCCu);
  const uint32_t t = (lo ^ (hi << 4)) & 0xF0F0F0F0u;
  lo ^= t;
  hi ^= t >> 4;
}

// Codes of coordinates 8n .. 8n+7 of one per-slot record (layout as stored at
// d < 128: widths 1, 2, 4 packed, width 3 a 2-bit plane then a 1-bit plane)
// as nibbles (coordinate 8n + j in bits 4j .. 4j+3).
template <int VB>
__device__ __forceinline__ uint32_t vg_row_nibbles(const uint8_t *row, int n) {
  if constexpr (VB == 4) {
    return *(const uint32_t *)(row + 4 * n);
  } else {
    uint32_t x = 0u;
    if constexpr (VB == 2 || VB == 3) {
      x = *(const uint16_t *)(row + 2 * n);                 // 2-bit units -> bits 4j, 4j+1
      x = (x | (x << 8)) & 0x00FF00FFu;
      x = (x | (x << 4)) & 0x0F0F0F0Fu;
      x = (x | (x << 2)) & 0x33333333u;
    }
    if constexpr (VB == 3 || VB == 1) {
      uint32_t h = row[VB == 3 ? 32 + n : n];              // bits -> bit 4j (+2 for width 3)
      h = (h | (h << 12)) & 0x000F000Fu;
      h = (h | (h << 6)) & 0x03030303u;
      h = (h | (h << 3)) & 0x11111111u;
      x |= VB == 3 ? h << 2 : h;
    }
    return x;
  }
}

// Emit the code groups of one wave tile of VT slots (tile start a multiple of
// VT, so of 4): rows = LDS rows of the tile's slots, RP bytes apart, holding
// per-slot records (16 VB bytes), or (NIB) one nibble per coordinate
// (coordinate c in bits 4 (c % 8) of byte-aligned word c / 8: 64 bytes);
// slots with rlo <= row < rhi are written, the others keep their stored bits.
// dst = the value codes at the tile's first slot.
template <int VB, int VT, int RP = 16 * VB, bool NIB = false>
__device__ __forceinline__ void vg_emit_codes(const uint8_t *rows, int rlo, int rhi, uint8_t *dst,
                                              int lane) {
  constexpr int PB = 4 * VB, QB = 64 * VB;
  constexpr uint32_t NM = VB == 4 ? 0xFFFFFFFFu : VB == 3 ? 0x77777777u : VB == 2 ? 0x33333333u
                                                                                  : 0x11111111u;
  // opaque per call: otherwise the lane-derived addresses are hoisted out of
  // the caller's tile loop and stay live through it (register pressure)
  asm volatile("" : "+v"(lane));
#pragma unroll 1
  for (int k = 0; k < VT / 16; ++k) {   // one piece at a time (few live registers)
    const int pi = lane + 64 * k;
    const int qd = pi >> 4, n = pi & 15;
    uint32_t N[4], V[4];
    int nv = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * qd + r;
      const bool ok = row >= rlo && row < rhi;
      N[r] = NIB ? *(const uint32_t *)(rows + row * RP + 4 * n) : vg_row_nibbles<VB>(rows + row * RP, n);
      V[r] = ok ? NM : 0u;
      nv += ok ? 1 : 0;
    }
    if (nv == 0) continue;
    uint32_t w[VB];
    vg_piece<VB>(N, w);
    uint32_t *p = (uint32_t *)(dst + qd * QB + n * PB);
    if (nv < 4) {
      // a group the call covers in part: keep the other slots' bits
      uint32_t m[VB];
      vg_piece<VB>(V, m);
#pragma unroll
      for (int i = 0; i < VB; ++i) w[i] = (p[i] & ~m[i]) | (w[i] & m[i]);
    }
    if constexpr (VB == 4) {
      *(u32x4 *)p = u32x4{w[0], w[1], w[2], w[3]};
    } else if constexpr (VB == 2) {
      *(u32x2 *)p = u32x2{w[0], w[1]};
    } else {
#pragma unroll
      for (int i = 0; i < VB; ++i) p[i] = w[i];
    }
  }
}

// Emit the sign groups of one wave tile of VT slots: srows = LDS sign records
// (16 bytes per slot, SP bytes apart; row k at byte k / 8 bit k % 8).  dst =
// the value signs at the tile's first slot.
template <int VT, int SP = 16>
__device__ __forceinline__ void vg_emit_signs(const uint8_t *srows, int rlo, int rhi, uint8_t *dst,
                                              int lane) {
  asm volatile("" : "+v"(lane));   // as in vg_emit_codes
#pragma unroll 1
  for (int k = 0; k < (VT * 2 + 63) / 64; ++k) {
    const int it = lane + 64 * k;
    if (it >= VT * 2) break;
    const int o = it >> 4, n = it & 15;   // octet, sketch rows 8n .. 8n+7
    uint32_t lo = 0u, hi = 0u, vm = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = 8 * o + e;
      const uint32_t by = srows[row * SP + n];
      if (e < 4) lo |= by << (8 * e);
      else hi |= by << (8 * (e - 4));
      vm |= (row >= rlo && row < rhi ? 1u : 0u) << e;
    }
    if (vm == 0u) continue;
    vg_transpose8(lo, hi);
    uint32_t *p = (uint32_t *)(dst + o * 128 + 8 * n);
    if (vm != 0xFFu) {
      const uint32_t mm = vm * 0x01010101u;
      lo = (p[0] & ~mm) | (lo & mm);
      hi = (p[1] & ~mm) | (hi & mm);
    }
    *(u32x2 *)p = u32x2{lo, hi};
  }
}

}  // namespace kvq
