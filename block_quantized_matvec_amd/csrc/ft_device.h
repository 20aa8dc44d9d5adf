// ft_device.h -- device-side building blocks shared by the gfx950 kernels:
// block format traits, the per-unit unpack + int8 dot4 core, activation preload
// and 64-lane reductions.
//
// A "unit" is the work of one lane on one row: 32 weights of one block (64 for
// Q4_K / Q5_K, whose lanes take both 32-element sub-blocks of one 64-element
// chunk so that one scale decode and one combine serve 64 weights).  The lane
// holds the matching activation codes (NW dwords of int8x4) in VGPRs, unpacks
// the unit's weight codes into the same dword order and takes integer dots with
// v_dot4_i32_i8.  A unit is cut into S "segments" whose elements share one
// weight scale and one activation block; the fp32 combine is, per segment,
//   acc += d_x * (wscale * I - wmin * B)
// with I the integer dot of raw codes and B the sum of the activation codes.
// (Q4_0's -8 and Q6_K's -32 code offsets enter through wmin.)  This is the
// keep-quant scheme of vllm.cpp PR #523 "grouped + non-grouped keep-quant expert
// GEMM" (What changed: superblock dots on an integer dot4 core), laid out for
// 64-lane wavefronts.  Block byte layouts are the public GGUF formats.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ft.h"

namespace ftk {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// format traits
//   BLK, BB   elements and bytes per block
//   UPB       units per block;  NW activation dwords per unit (4 codes each)
//   S         segments per unit; SUB elements per exported integer partial
//   act_elem(ui, j)  element (within the block) of the first code of dword j
//   seg_of(j)        segment of dword j
// ---------------------------------------------------------------------------
template <int F> struct Fmt;

// Q4_0: fp16 d @0, qs[16] @2; element e<16 low nibble of qs[e], else high nibble
// of qs[e-16]; w = d*(n-8).  One unit, one segment.
template <> struct Fmt<FT_Q4_0> {
  static constexpr int BLK = 32, BB = 18, UPB = 1, NW = 8, S = 1, SUB = 32;
  static constexpr bool XF1 = false;      // see Fmt<FT_Q4_K>
  static constexpr bool HAS_MIN = true;   // the -8 offset, as wmin = 8d
  static constexpr int CODE_OFF = 8;      // exported partials use n - 8
  __device__ static int act_elem(int, int j) { return 4 * j; }
  __device__ static constexpr int seg_of(int) { return 0; }
};
// Q8_0: fp16 d @0, int8 qs[32] @2; w = d*q.
template <> struct Fmt<FT_Q8_0> {
  static constexpr int BLK = 32, BB = 34, UPB = 1, NW = 8, S = 1, SUB = 32;
  static constexpr bool XF1 = false;
  static constexpr bool HAS_MIN = false;
  static constexpr int CODE_OFF = 0;
  __device__ static int act_elem(int, int j) { return 4 * j; }
  __device__ static constexpr int seg_of(int) { return 0; }
};
// MXFP4: E8M0 e @0, qs[16] @1 (nibble order as Q4_0); w = v2 * 2^(e-128) with v2
// twice the E2M1 value (an integer in [-12, 12]).
template <> struct Fmt<FT_MXFP4> {
  static constexpr int BLK = 32, BB = 17, UPB = 1, NW = 8, S = 1, SUB = 32;
  static constexpr bool XF1 = false;
  static constexpr bool HAS_MIN = false;
  static constexpr int CODE_OFF = 0;
  __device__ static int act_elem(int, int j) { return 4 * j; }
  __device__ static constexpr int seg_of(int) { return 0; }
};
// Q4_K: d @0, dmin @2, scales[12] @4, qs[128] @16.  Element e = 64c + 32h + l is
// nibble h of qs[32c+l]; sub-block j = 2c+h.  Unit c covers qs[32c .. 32c+31]:
// dwords 0-7 are its low nibbles (sub-block 2c), dwords 8-15 its high nibbles
// (sub-block 2c+1).  XF1: the high nibbles are taken as the int8 bytes
// (q & 0xF0) ^ 0x80 = 16*hi - 128 (one bitwise op per dword); their dot D relates
// to the true one by I = (D + 128*B)/16, folded into the activation scale (dx/16)
// and the min term (wmin - 8*wscale).
template <> struct Fmt<FT_Q4_K> {
  static constexpr int BLK = 256, BB = 144, UPB = 4, NW = 16, S = 2, SUB = 32;
  static constexpr bool XF1 = true;
  static constexpr bool HAS_MIN = true;
  static constexpr int CODE_OFF = 0;
  __device__ static int act_elem(int ui, int j) { return 64 * ui + (j < 8 ? 4 * j : 32 + 4 * (j - 8)); }
  __device__ static constexpr int seg_of(int j) { return j >> 3; }
};
// Q5_K: d @0, dmin @2, scales[12] @4, qh[32] @16, qs[128] @48; as Q4_K with the
// fifth bit of element 64c+32h+l in bit (2c+h) of qh[l].
template <> struct Fmt<FT_Q5_K> {
  static constexpr int BLK = 256, BB = 176, UPB = 4, NW = 16, S = 2, SUB = 32;
  static constexpr bool XF1 = false;
  static constexpr bool HAS_MIN = true;
  static constexpr int CODE_OFF = 0;
  __device__ static int act_elem(int ui, int j) { return Fmt<FT_Q4_K>::act_elem(ui, j); }
  __device__ static constexpr int seg_of(int j) { return j >> 3; }
};
// Q6_K: ql[128] @0, qh[64] @128, int8 scales[16] @192, fp16 d @208.  Element
// e = 128g + 32r + l: low 4 bits from ql[64g + 32(r&1) + l] (low nibble for r<2,
// high for r>=2), top 2 bits = bits 2r..2r+1 of qh[32g + l]; w = d*sc[e/16]*(q6-32).
// Unit ui = 4g + (l0/8) covers l in [l0, l0+8) for all four r: dwords 2r, 2r+1.
template <> struct Fmt<FT_Q6_K> {
  static constexpr int BLK = 256, BB = 210, UPB = 8, NW = 8, S = 4, SUB = 16;
  static constexpr bool XF1 = false;
  static constexpr bool HAS_MIN = true;   // the -32 offset, as wmin = 32*d*sc
  static constexpr int CODE_OFF = 32;
  __device__ static int act_elem(int ui, int j) {
    return 128 * (ui >> 2) + 32 * (j >> 1) + 8 * (ui & 3) + 4 * (j & 1);
  }
  __device__ static constexpr int seg_of(int j) { return j >> 1; }
};

// Q2_K: scales[16] @0 (low nibble scale, high nibble min of 16-element sub-block
// j), qs[64] @16, fp16 d @80, dmin @82.  Element e = 128g + 32r + l is bits
// 2r..2r+1 of qs[32g + l]; w = d*sc_j*q - dmin*m_j with j = e/16.  Unit ui = 4g + r
// covers that (g, r): dwords 0-3 are sub-block 2ui, dwords 4-7 sub-block 2ui+1.
template <> struct Fmt<FT_Q2_K> {
  static constexpr int BLK = 256, BB = 84, UPB = 8, NW = 8, S = 2, SUB = 16;
  static constexpr bool XF1 = false;
  static constexpr bool HAS_MIN = true;
  static constexpr int CODE_OFF = 0;
  __device__ static int act_elem(int ui, int j) { return 32 * ui + 4 * j; }
  __device__ static constexpr int seg_of(int j) { return j >> 2; }
};
// Q3_K: hmask[32] @0, qs[64] @32, scales[12] @96, fp16 d @108.  Codes as Q2_K plus
// a third bit, bit 4g + r of hmask[l]; the unit carries q + 4 (0..7) and the -4
// offset enters through wmin = 4 * wscale.  Signed 6-bit scale of sub-block j,
// stored plus 32: low four bits in the low (j < 8) or high (j >= 8) nibble of
// scales[j % 8], top two bits at bit 2(j/4) of scales[8 + j % 4].
template <> struct Fmt<FT_Q3_K> {
  static constexpr int BLK = 256, BB = 110, UPB = 8, NW = 8, S = 2, SUB = 16;
  static constexpr bool XF1 = false;
  static constexpr bool HAS_MIN = true;
  static constexpr int CODE_OFF = 4;
  __device__ static int act_elem(int ui, int j) { return 32 * ui + 4 * j; }
  __device__ static constexpr int seg_of(int j) { return j >> 2; }
};

// Q4_1: fp16 d @0, fp16 m @2, qs[16] @4 (nibble order as Q4_0); w = d*n + m, the
// offset entering as wmin = -m.  Q5_0: d @0, qh @2 (32 bits, bit e the fifth bit of
// element e), qs[16] @6; w = d*(q-16), the -16 as wmin = 16d.  Q5_1: d @0, m @2,
// qh @4, qs[16] @8; w = d*q + m.  One unit, one segment, as Q4_0.
template <int F> struct FmtLegacy {
  static constexpr int BLK = 32, UPB = 1, NW = 8, S = 1, SUB = 32;
  static constexpr bool XF1 = false;
  static constexpr bool HAS_MIN = true;
  __device__ static int act_elem(int, int j) { return 4 * j; }
  __device__ static constexpr int seg_of(int) { return 0; }
};
template <> struct Fmt<FT_Q4_1> : FmtLegacy<FT_Q4_1> { static constexpr int BB = 20, CODE_OFF = 0; };
template <> struct Fmt<FT_Q5_0> : FmtLegacy<FT_Q5_0> { static constexpr int BB = 22, CODE_OFF = 16; };
template <> struct Fmt<FT_Q5_1> : FmtLegacy<FT_Q5_1> { static constexpr int BB = 24, CODE_OFF = 0; };

template <int A> struct Act;
template <> struct Act<FT_Q8_1> { static constexpr int BLK = 32, BB = 36; };
template <> struct Act<FT_Q8_K> { static constexpr int BLK = 256, BB = 292; };

// units in a row of k elements (host and device)
template <int F>
__host__ __device__ constexpr int64_t units_in_row(int64_t k) {
  return k / Fmt<F>::BLK * Fmt<F>::UPB;
}

// ---------------------------------------------------------------------------
// scalar helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float h2f(uint32_t bits16) {
  _Float16 h;
  uint16_t b = (uint16_t)bits16;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}
__device__ __forceinline__ uint32_t f2h_bits(float f) {  // round to nearest even
  _Float16 h = (_Float16)f;
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}
// 2^(e-128) for an E8M0 byte, built from its bits (exact, subnormals for e < 2)
__device__ __forceinline__ float e8m0_half(uint32_t e) {
  uint32_t bits = e >= 2 ? (e - 1) << 23 : (0x00400000u >> (1 - e));
  return __uint_as_float(bits);
}
// Index of the calling wave in its workgroup, as a wave-uniform (SGPR) value.  The
// compiler cannot tell that threadIdx.x / 64 is the same in every lane; anything
// derived from it (row shares, loop bounds, load addresses) would otherwise be
// per-lane VALU work under exec-masked branches.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// ---------------------------------------------------------------------------
// byte-addressed readers over a dword array (LDS tile or global blocks).
// u32(off) returns the 4 bytes at any byte offset.
// ---------------------------------------------------------------------------
template <typename P>
struct Reader {
  P base;  // const uint32_t* in LDS (address space inferred) or global
  __device__ __forceinline__ uint32_t u32(uint32_t off) const {
    uint32_t lo = base[off >> 2], hi = base[(off >> 2) + 1];
    return __builtin_amdgcn_alignbyte(hi, lo, off & 3);
  }
  template <int N>
  __device__ __forceinline__ void dwords(uint32_t off, uint32_t (&o)[N]) const {
    const uint32_t w0 = off >> 2, sh = off & 3;
    uint32_t prev = base[w0];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      uint32_t nx = base[w0 + i + 1];
      o[i] = __builtin_amdgcn_alignbyte(nx, prev, sh);
      prev = nx;
    }
  }
  // off must be 16-byte aligned; N a multiple of 4
  template <int N>
  __device__ __forceinline__ void dwords16(uint32_t off, uint32_t (&o)[N]) const {
    const u32x4* b = (const u32x4*)base;
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const u32x4 v = b[(off >> 4) + i];
      o[4 * i] = v.x;
      o[4 * i + 1] = v.y;
      o[4 * i + 2] = v.z;
      o[4 * i + 3] = v.w;
    }
  }
  __device__ __forceinline__ uint32_t u16(uint32_t off) const { return (u32(off)) & 0xFFFFu; }
  __device__ __forceinline__ uint32_t u8(uint32_t off) const {
    return (base[off >> 2] >> (8 * (off & 3))) & 0xFFu;
  }
};

// ---------------------------------------------------------------------------
// unit unpack: weight codes in activation dword order + per-segment scale/min
// ---------------------------------------------------------------------------
template <int F> struct Unit {
  uint32_t w[Fmt<F>::NW];
  float ws[Fmt<F>::S];
  float wm[Fmt<F>::S];
};

// K-quant 6-bit scale and min of sub-block j from the three header dwords
// h0 = scales[0..3], h1 = scales[4..7], h2 = scales[8..11] (element-wise use).
__device__ __forceinline__ void kq_scale_min(uint32_t h0, uint32_t h1, uint32_t h2, int j,
                                             uint32_t& sc, uint32_t& m) {
  if (j < 4) {
    sc = (h0 >> (8 * j)) & 63;
    m = (h1 >> (8 * j)) & 63;
  } else {
    const int jj = j - 4;
    const uint32_t b8 = (h2 >> (8 * jj)) & 0xFF;
    sc = (b8 & 15) | (((h0 >> (8 * jj + 6)) & 3) << 4);
    m = (b8 >> 4) | (((h1 >> (8 * jj + 6)) & 3) << 4);
  }
}

// All eight 6-bit scales and mins of a K-quant superblock, four per dword:
// sc_lo bytes = sc_0..3, sc_hi = sc_4..7, m_lo = m_0..3, m_hi = m_4..7.
// (Sub-blocks 4-7 keep their low four bits in bytes 8-11 -- scale in the low
// nibble, min in the high nibble -- and their top two bits in the spare top bits
// of bytes 0-3 (scale) and 4-7 (min).)
__device__ __forceinline__ void kq_unpack_scales(uint32_t h0, uint32_t h1, uint32_t h2, uint32_t& sc_lo,
                                                 uint32_t& sc_hi, uint32_t& m_lo, uint32_t& m_hi) {
  sc_lo = h0 & 0x3F3F3F3Fu;
  m_lo = h1 & 0x3F3F3F3Fu;
  sc_hi = (h2 & 0x0F0F0F0Fu) | ((h0 >> 2) & 0x30303030u);
  m_hi = ((h2 >> 4) & 0x0F0F0F0Fu) | ((h1 >> 2) & 0x30303030u);
}

// K-quant header (d|dmin, scales) -> wscale / wmin of the two sub-blocks 2c, 2c+1
// of unit c: bytes 2(c&1), 2(c&1)+1 of the lo (c < 2) or hi (c >= 2) packed dwords.
__device__ __forceinline__ void kq_header(uint32_t h_ddm, uint32_t h0, uint32_t h1, uint32_t h2, int c,
                                          float (&ws)[2], float (&wm)[2]) {
  const float d = h2f(h_ddm & 0xFFFF), dmin = h2f(h_ddm >> 16);
  uint32_t sc_lo, sc_hi, m_lo, m_hi;
  kq_unpack_scales(h0, h1, h2, sc_lo, sc_hi, m_lo, m_hi);
  const uint32_t sh = 16u * (uint32_t)(c & 1);
  const uint32_t sc = (c >= 2 ? sc_hi : sc_lo) >> sh;
  const uint32_t m = (c >= 2 ? m_hi : m_lo) >> sh;
  ws[0] = d * (float)(sc & 0xFF);
  ws[1] = d * (float)((sc >> 8) & 0xFF);
  wm[0] = dmin * (float)(m & 0xFF);
  wm[1] = dmin * (float)((m >> 8) & 0xFF);
}

// bits 0..3 of h to bit 0 of bytes 0..3 (the fifth bits of four consecutive elements)
__device__ __forceinline__ uint32_t spread4(uint32_t h) {
  h &= 15u;
  return (h | (h << 7) | (h << 14) | (h << 21)) & 0x01010101u;
}

// E2M1 codes (one per byte, 0..15) -> twice their value as int8, via byte permutes:
// magnitudes 0,1,2,3,4,6,8,12 for codes 0..7; codes 8..15 are the negatives.
__device__ __forceinline__ uint32_t e2m1x2_bytes(uint32_t c) {
  const uint32_t sel = c & 0x07070707u;
  const uint32_t pos = __builtin_amdgcn_perm(0x0C080604u, 0x03020100u, sel);
  const uint32_t neg = __builtin_amdgcn_perm(0xF4F8FAFCu, 0xFDFEFF00u, sel);
  const uint32_t sb = c & 0x08080808u;
  const uint32_t mask = (sb << 5) - (sb >> 3);  // 0xFF in every byte whose code is negative
  return (neg & mask) | (pos & ~mask);
}

// K-quant unit c from registers: header h (d|dmin, 12 scale bytes), the 32 nibble
// bytes q of chunk c and, for Q5_K, the 32 fifth-bit bytes qh.
template <int F>
__device__ __forceinline__ void kq_unit(const uint32_t (&h)[4], const uint32_t (&q)[8], const uint32_t (&qh)[8],
                                        int c, Unit<F>& u) {
  kq_header(h[0], h[1], h[2], h[3], c, u.ws, u.wm);
  if constexpr (F == FT_Q4_K) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      u.w[m] = q[m] & 0x0F0F0F0Fu;
      u.w[8 + m] = (q[m] & 0xF0F0F0F0u) ^ 0x80808080u;   // 16*hi - 128 as int8
    }
    u.wm[1] = fmaf(-8.0f, u.ws[1], u.wm[1]);
  } else {
    const uint32_t hb = 2u * (uint32_t)c;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      u.w[m] = (q[m] & 0x0F0F0F0Fu) | (((qh[m] >> hb) & 0x01010101u) << 4);
      u.w[8 + m] = ((q[m] >> 4) & 0x0F0F0F0Fu) | (((qh[m] >> (hb + 1)) & 0x01010101u) << 4);
    }
  }
}

// A16: the block's offset is 16-byte aligned in the reader (K-quant rows always
// are: 144- and 176-byte blocks in 16-byte-aligned rows).
template <int F, bool A16, typename R>
__device__ __forceinline__ void unpack_unit(const R& rd, uint32_t bo, int ui, Unit<F>& u) {
  if constexpr (F == FT_Q4_0) {
    const float d = h2f(rd.u16(bo));
    uint32_t q[4];
    rd.template dwords<4>(bo + 2, q);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      u.w[m] = q[m] & 0x0F0F0F0Fu;
      u.w[4 + m] = (q[m] >> 4) & 0x0F0F0F0Fu;
    }
    u.ws[0] = d;
    u.wm[0] = 8.0f * d;
  } else if constexpr (F == FT_Q8_0) {
    u.ws[0] = h2f(rd.u16(bo));
    u.wm[0] = 0.0f;
    rd.template dwords<8>(bo + 2, u.w);
  } else if constexpr (F == FT_MXFP4) {
    u.ws[0] = e8m0_half(rd.u8(bo));
    u.wm[0] = 0.0f;
    uint32_t q[4];
    rd.template dwords<4>(bo + 1, q);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      u.w[m] = e2m1x2_bytes(q[m] & 0x0F0F0F0Fu);
      u.w[4 + m] = e2m1x2_bytes((q[m] >> 4) & 0x0F0F0F0Fu);
    }
  } else if constexpr (F == FT_Q4_K || F == FT_Q5_K) {
    uint32_t h[4], q[8], qh[8];
    constexpr uint32_t QOFF = F == FT_Q4_K ? 16 : 48;
    if constexpr (A16) {
      rd.template dwords16<4>(bo, h);
      rd.template dwords16<8>(bo + QOFF + 32 * ui, q);
      if constexpr (F == FT_Q5_K) rd.template dwords16<8>(bo + 16, qh);
    } else {
      rd.template dwords<4>(bo, h);
      rd.template dwords<8>(bo + QOFF + 32 * ui, q);
      if constexpr (F == FT_Q5_K) rd.template dwords<8>(bo + 16, qh);
    }
    kq_unit<F>(h, q, qh, ui, u);
  } else if constexpr (F == FT_Q4_1 || F == FT_Q5_0 || F == FT_Q5_1) {
    constexpr uint32_t QO = F == FT_Q4_1 ? 4 : F == FT_Q5_0 ? 6 : 8;   // first nibble byte
    uint32_t q[4];
    rd.template dwords<4>(bo + QO, q);
    const float d = h2f(rd.u16(bo));
    uint32_t qh = 0;
    if constexpr (F != FT_Q4_1) qh = rd.u32(bo + QO - 4);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      u.w[m] = q[m] & 0x0F0F0F0Fu;
      u.w[4 + m] = (q[m] >> 4) & 0x0F0F0F0Fu;
      if constexpr (F != FT_Q4_1) {
        u.w[m] |= spread4(qh >> (4 * m)) << 4;
        u.w[4 + m] |= spread4(qh >> (16 + 4 * m)) << 4;
      }
    }
    u.ws[0] = d;
    u.wm[0] = F == FT_Q5_0 ? 16.0f * d : -h2f(rd.u16(bo + 2));
  } else if constexpr (F == FT_Q2_K || F == FT_Q3_K) {
    const int g = ui >> 2, r = ui & 3;
    uint32_t q[8];
    rd.template dwords<8>(bo + (F == FT_Q2_K ? 16 : 32) + 32 * g, q);
    if constexpr (F == FT_Q2_K) {
#pragma unroll
      for (int m = 0; m < 8; ++m) u.w[m] = (q[m] >> (2 * r)) & 0x03030303u;
      const uint32_t sc = rd.u16(bo + 2 * ui);   // scale|min bytes of sub-blocks 2ui, 2ui+1
      const uint32_t dd = rd.u32(bo + 80);
      const float d = h2f(dd & 0xFFFF), dmin = h2f(dd >> 16);
      u.ws[0] = d * (float)(sc & 15);
      u.wm[0] = dmin * (float)((sc >> 4) & 15);
      u.ws[1] = d * (float)((sc >> 8) & 15);
      u.wm[1] = dmin * (float)(sc >> 12);
    } else {
      uint32_t hm[8];
      rd.template dwords<8>(bo, hm);
      const int hb = 4 * g + r;
#pragma unroll
      for (int m = 0; m < 8; ++m)
        u.w[m] = ((q[m] >> (2 * r)) & 0x03030303u) | (((hm[m] >> hb) & 0x01010101u) << 2);
      const float d = h2f(rd.u16(bo + 108));
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int j = 2 * ui + s;
        const uint32_t lo = (rd.u8(bo + 96 + (j & 7)) >> (j < 8 ? 0 : 4)) & 15;
        const uint32_t hi = (rd.u8(bo + 104 + (j & 3)) >> (2 * (j >> 2))) & 3;
        u.ws[s] = d * (float)((int)(lo | (hi << 4)) - 32);
        u.wm[s] = 4.0f * u.ws[s];
      }
    }
  } else {  // Q6_K
    const int g = ui >> 2, l0 = 8 * (ui & 3);
    uint32_t qa[2], qb[2], qh[2];
    rd.template dwords<2>(bo + 64 * g + l0, qa);        // r = 0 (low nibbles), r = 2 (high)
    rd.template dwords<2>(bo + 64 * g + 32 + l0, qb);   // r = 1 (low nibbles), r = 3 (high)
    rd.template dwords<2>(bo + 128 + 32 * g + l0, qh);
    const float d = h2f(rd.u16(bo + 208));
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      u.w[0 + m] = (qa[m] & 0x0F0F0F0Fu) | ((qh[m] & 0x03030303u) << 4);
      u.w[2 + m] = (qb[m] & 0x0F0F0F0Fu) | (((qh[m] >> 2) & 0x03030303u) << 4);
      u.w[4 + m] = ((qa[m] >> 4) & 0x0F0F0F0Fu) | (((qh[m] >> 4) & 0x03030303u) << 4);
      u.w[6 + m] = ((qb[m] >> 4) & 0x0F0F0F0Fu) | (((qh[m] >> 6) & 0x03030303u) << 4);
    }
    // scales of the four segments: sc[8g + 2r + l0/16]
    const uint32_t sbase = bo + 192 + 8 * g + (l0 >> 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float sc = (float)(int8_t)rd.u8(sbase + 2 * r);
      u.ws[r] = d * sc;
      u.wm[r] = 32.0f * u.ws[r];
    }
  }
}

// ---------------------------------------------------------------------------
// activations of one unit position, held in VGPRs
// ---------------------------------------------------------------------------
template <int F> struct ActUnit {
  uint32_t x[Fmt<F>::NW];      // int8x4 codes, dword j <-> Fmt<F>::act_elem(ui, j)
  float dx[Fmt<F>::S];         // activation scale of each segment (dx/16 for XF1's segment 1)
  float dxb[Fmt<F>::S];        // true dx * (sum of the segment's codes)
  int bsum[Fmt<F>::S];         // sum of the segment's codes
};

// first dword of segment s
template <int F>
__device__ __forceinline__ constexpr int seg_first(int s) {
  int j0 = 0;
  for (int j = Fmt<F>::NW - 1; j >= 0; --j)
    if (Fmt<F>::seg_of(j) == s) j0 = j;
  return j0;
}

// Load the activation codes of unit (block b, unit ui) of one token row, in two
// steps: load_act_raw issues the loads only (codes into x, the raw scale bits of
// each segment parked in bsum), finish_act_unit derives the rest once they have
// arrived (so that other loads can be issued between the two), and zeroes the
// unit when !valid.  xrow: that token's activation blocks (dword aligned).
template <int F, int A>
__device__ __forceinline__ void load_act_raw(const uint8_t* __restrict__ xrow, int b, int ui, ActUnit<F>& a) {
  constexpr int S = Fmt<F>::S, NW = Fmt<F>::NW;
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const int e = b * Fmt<F>::BLK + Fmt<F>::act_elem(ui, j);
    const int ab = e / Act<A>::BLK, pos = e % Act<A>::BLK;
    a.x[j] = *(const uint32_t*)(xrow + (size_t)ab * Act<A>::BB + 4 + pos);
  }
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e = b * Fmt<F>::BLK + Fmt<F>::act_elem(ui, seg_first<F>(s));
    const uint8_t* ab = xrow + (size_t)(e / Act<A>::BLK) * Act<A>::BB;
    if (A == FT_Q8_1) a.bsum[s] = (int)*(const uint16_t*)ab;
    else a.bsum[s] = *(const int*)ab;
  }
}

template <int F, int A>
__device__ __forceinline__ void finish_act_unit(ActUnit<F>& a, bool valid) {
  constexpr int S = Fmt<F>::S, NW = Fmt<F>::NW;
  float dx[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const float d = A == FT_Q8_1 ? h2f((uint32_t)a.bsum[s]) : __int_as_float(a.bsum[s]);
    dx[s] = valid ? d : 0.0f;
    a.bsum[s] = 0;
  }
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    a.x[j] = valid ? a.x[j] : 0u;
    a.bsum[Fmt<F>::seg_of(j)] = dot4(a.x[j], 0x01010101u, a.bsum[Fmt<F>::seg_of(j)]);
  }
#pragma unroll
  for (int s = 0; s < S; ++s) {
    a.dxb[s] = dx[s] * (float)a.bsum[s];
    a.dx[s] = (Fmt<F>::XF1 && s == 1) ? dx[s] * 0.0625f : dx[s];
  }
}

template <int F, int A>
__device__ __forceinline__ void load_act_unit(const uint8_t* __restrict__ xrow, int b, int ui, ActUnit<F>& a) {
  load_act_raw<F, A>(xrow, b, ui, a);
  finish_act_unit<F, A>(a, true);
}

// true integer dot of segment s from the raw dot D of the unpacked codes
template <int F>
__device__ __forceinline__ int seg_true_dot(int s, int D, int bsum) {
  return (Fmt<F>::XF1 && s == 1) ? (D + 128 * bsum) >> 4 : D;
}

template <int F>
__device__ __forceinline__ void zero_act_unit(ActUnit<F>& a) {
#pragma unroll
  for (int j = 0; j < Fmt<F>::NW; ++j) a.x[j] = 0;
#pragma unroll
  for (int s = 0; s < Fmt<F>::S; ++s) { a.dx[s] = 0.f; a.dxb[s] = 0.f; a.bsum[s] = 0; }
}

// Integer dot of each segment of a unit against one token's codes.
template <int F>
__device__ __forceinline__ void unit_dots(const Unit<F>& u, const ActUnit<F>& a, int (&I)[Fmt<F>::S]) {
#pragma unroll
  for (int s = 0; s < Fmt<F>::S; ++s) I[s] = 0;
#pragma unroll
  for (int j = 0; j < Fmt<F>::NW; ++j) I[Fmt<F>::seg_of(j)] = dot4(u.w[j], a.x[j], I[Fmt<F>::seg_of(j)]);
}

// fp32 combine of one unit for one token.
template <int F>
__device__ __forceinline__ float unit_combine(const Unit<F>& u, const ActUnit<F>& a, float acc) {
  int I[Fmt<F>::S];
  unit_dots<F>(u, a, I);
#pragma unroll
  for (int s = 0; s < Fmt<F>::S; ++s) {
    acc = fmaf(a.dx[s] * (float)I[s], u.ws[s], acc);
    if (Fmt<F>::HAS_MIN) acc = fmaf(-u.wm[s], a.dxb[s], acc);
  }
  return acc;
}

// ---------------------------------------------------------------------------
// activation quantizers (shared by the standalone quantize kernels and the fused
// prologues of the MoE kernels, so both are bit-identical).
// amax, d = amax/127 (fp16 for Q8_1, fp32 for Q8_K), q = clamp(round half away
// from zero of x/d against the stored d, +-127), IEEE correctly rounded division.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int q8_code(float v, float d) {
  // branch-free (the code is 0 for d = 0), so a block's divisions can overlap
  const float rq = roundf(v / (d == 0.0f ? 1.0f : d));
  const int q = rq > 127.0f ? 127 : (rq < -127.0f ? -127 : (int)rq);
  return d == 0.0f ? 0 : q;
}

// The same codes for N elements of one scale, without a division per element.
// While |v / d| < 128, t = v * rcp(d) is within 1.5 * 2^-16 of v / d (v_rcp_f32
// within 1 ulp, then the product's rounding) and the correctly rounded quotient
// within 2^-18 of it, so the two round to the same integer unless t lies within
// 2^-14 of a half-integer; larger quotients clamp to 127 either way.  A lane with
// such an element, or with a scale outside [2^-100, 2^100] (zero included), takes
// q8_code's division for all N.  Away from half-integers round-half-even
// (v_rndne) and round-half-away agree.
template <int N>
__device__ __forceinline__ void q8_codes(const float (&v)[N], float d, int (&q)[N]) {
  const float r = __builtin_amdgcn_rcpf(d);
  bool slow = !(d >= 0x1p-100f && d <= 0x1p100f);
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const float t = v[j] * r;
    slow |= fabsf(__builtin_amdgcn_fractf(t) - 0.5f) <= 0x1p-14f;
    const int k = (int)__builtin_rintf(t);
    q[j] = k > 127 ? 127 : (k < -127 ? -127 : k);
  }
  if (slow) {
#pragma unroll
    for (int j = 0; j < N; ++j) q[j] = q8_code(v[j], d);
  }
}

// ---------------------------------------------------------------------------
// 64-lane reductions
// ---------------------------------------------------------------------------
// value of the partner lane at xor-distance S (S = 1, 2: quad permutes; 4, 8:
// half-row / row mirrors, which pair lanes across the same bit; 16, 32: LDS
// permute).
template <int S>
__device__ __forceinline__ float xchg(float v) {
  const int i = __float_as_int(v);
  int r;
  if constexpr (S == 1) r = __builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, false);       // quad_perm [1,0,3,2]
  else if constexpr (S == 2) r = __builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  else if constexpr (S == 4) r = __builtin_amdgcn_mov_dpp(i, 0x141, 0xF, 0xF, false); // row_half_mirror
  else if constexpr (S == 8) r = __builtin_amdgcn_mov_dpp(i, 0x140, 0xF, 0xF, false); // row_mirror
  else r = __shfl_xor(i, S, 64);
  return __int_as_float(r);
}

// Block quantizers over several elements per lane; the lanes of one block combine
// their amax (and Q8_1's code sum) with DPP moves.  Max and integer sums do not
// depend on the order of reduction, so any lane split gives the same block.
// Q8_1: 4 aligned lanes per 32-element block, lane l4 = 0..3 holds elements
// 8*l4 .. 8*l4+7.  The 4 lanes call it together; ob: the 36-byte block.
__device__ __forceinline__ void q8_1_part(const float (&v)[8], int l4, uint8_t* ob) {
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(v[j]));
  a = fmaxf(a, xchg<1>(a));
  a = fmaxf(a, xchg<2>(a));
  uint32_t dh = f2h_bits(a / 127.0f);
  const float d = h2f(dh);
  uint32_t w[2] = {0u, 0u};
  int s = 0;
  int qc[8];
  q8_codes<8>(v, d, qc);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = qc[j];
    s += q;
    w[j >> 2] |= ((uint32_t)(uint8_t)(int8_t)q) << (8 * (j & 3));
  }
  s += __float_as_int(xchg<1>(__int_as_float(s)));
  s += __float_as_int(xchg<2>(__int_as_float(s)));
  uint32_t* o = (uint32_t*)(ob + 4 + 8 * l4);
  o[0] = w[0];
  o[1] = w[1];
  if (l4 == 0) {
    if (d == 0.0f) dh = 0;
    const uint32_t sh = f2h_bits(d * (float)s);
    *(uint32_t*)ob = dh | (sh << 16);
  }
}

// Q8_K: 16 aligned lanes (one DPP row) per 256-element block, lane l16 holds
// elements 16*l16 .. 16*l16+15, i.e. exactly one 16-element bsum group.  Returns
// the lane's 16 codes (w), their sum (s) and the block scale (d).
__device__ __forceinline__ void q8_k_codes(const float (&v)[16], uint32_t (&w)[4], int& s, float& d) {
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(v[j]));
  a = fmaxf(a, xchg<1>(a));
  a = fmaxf(a, xchg<2>(a));
  a = fmaxf(a, xchg<4>(a));   // row half-mirror: quad 0 <-> quad 1 of each 8
  a = fmaxf(a, xchg<8>(a));   // row mirror: half 0 <-> half 1
  d = a / 127.0f;
  s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = 0u;
  int qc[16];
  q8_codes<16>(v, d, qc);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int q = qc[j];
    s += q;
    w[j >> 2] |= ((uint32_t)(uint8_t)(int8_t)q) << (8 * (j & 3));
  }
}
// ... and stores the lane's part of the 292-byte block at ob
__device__ __forceinline__ void q8_k_store(const uint32_t (&w)[4], int s, float d, int l16, uint8_t* ob) {
  uint32_t* o = (uint32_t*)(ob + 4 + 16 * l16);
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = w[i];
  *(int16_t*)(ob + 260 + 2 * l16) = (int16_t)s;
  if (l16 == 0) *(float*)ob = d;
}
__device__ __forceinline__ void q8_k_part(const float (&v)[16], int l16, uint8_t* ob) {
  uint32_t w[4];
  int s;
  float d;
  q8_k_codes(v, w, s, d);
  q8_k_store(w, s, d, l16, ob);
}

// ---------------------------------------------------------------------------
// router (ds4 PR #656 Summary; the routing semantics as read from the pages):
// one wave per token.  Top-k with ties going to the lower expert index, then a
// softmax over the selected logits in slot order.
//  * logits become order-preserving unsigned keys (-0 first folded into +0, so
//    that they tie as they compare equal);
//  * k rounds of a wave-wide arg-max: round r takes the largest key not yet
//    taken, the lowest expert index among equal keys, as slot r;
//  * slot r's weight is exp(l_r - l_0) / sum_q exp(l_q - l_0), the sum taken in
//    slot order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t route_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float route_val(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// the maximum of v over the wave, in every lane
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));   // row_mirror
  const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);           // (own, partner) either way
  v = max(r16[0], r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(r32[0], r32[1]);
}

// One token's routing by one wave, in two calls so that the logits can be in
// flight while the wave does other work: route_load reads them (lane l holds
// experts l*MAXE .. l*MAXE + MAXE - 1, so expert order is lane order), and
// route_select picks the winners; ids[0..k) / w[0..k) receive them in slot order
// (LDS or global).  Each lane keeps the best of its keys not yet taken (higher
// key, then lower expert); a round is one wave max over those, the lowest lane
// holding it wins, and only that lane looks at its keys again.
template <int MAXE>
__device__ __forceinline__ void route_load(const float* __restrict__ l, int n_expert, int lane, float (&raw)[MAXE]) {
#pragma unroll
  for (int i = 0; i < MAXE; ++i) {
    const int e = lane * MAXE + i;
    raw[i] = e < n_expert ? l[e] : 0.0f;
  }
}
template <int MAXE>   // logits per lane (n_expert <= 64 * MAXE)
__device__ __forceinline__ void route_select(const float (&raw)[MAXE], int n_expert, int topk, int lane,
                                             int32_t* ids, float* w) {
  uint32_t key[MAXE];
  uint32_t open = 0;               // bit i: key[i] is an expert not yet taken
#pragma unroll
  for (int i = 0; i < MAXE; ++i) {
    key[i] = route_key(raw[i]);
    if (lane * MAXE + i < n_expert) open |= 1u << i;
  }
  // this lane's best open key (bk) and its index (bs); bs = -1: none open
  uint32_t bk = 0;
  int bs = -1;
  auto rescan = [&]() {
    bk = 0;
    bs = -1;
#pragma unroll
    for (int i = 0; i < MAXE; ++i) {
      const bool better = ((open >> i) & 1) && (bs < 0 || key[i] > bk);
      bk = better ? key[i] : bk;
      bs = better ? i : bs;
    }
  };
  rescan();
  uint32_t my_key = 0;             // lane r < k: slot r's key and expert
  int my_idx = 0;
  for (int r = 0; r < topk; ++r) {
    const uint32_t mx = wave_umax(bk);
    const uint64_t b = __ballot(bs >= 0 && bk == mx);
    const int wl = (int)__builtin_ctzll(b);
    const int ws = __builtin_amdgcn_readlane(bs, wl);
    if (lane == r) {
      my_key = mx;
      my_idx = wl * MAXE + ws;
    }
    if (lane == wl) {
      open &= ~(1u << ws);
      rescan();
    }
  }
  const uint32_t top = __builtin_amdgcn_readlane(my_key, 0);
  const float ex = lane < topk ? expf(route_val(my_key) - route_val(top)) : 0.0f;
  float den = 0.0f;
  for (int q = 0; q < topk; ++q) den += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), q));
  if (lane < topk) {
    ids[lane] = my_idx;
    w[lane] = ex / den;
  }
}
template <int MAXE>
__device__ __forceinline__ void route_token(const float* __restrict__ l, int n_expert, int topk, int lane,
                                            int32_t* ids, float* w) {
  float raw[MAXE];
  route_load<MAXE>(l, n_expert, lane, raw);
  route_select<MAXE>(raw, n_expert, topk, lane, ids, w);
}

// The same selection by a whole workgroup of NT threads, for the t tokens of a
// chunk (ne = t * n_expert keys, element q = token q / n_expert).  Each (token,
// expert) gets a 64-bit key: the order-preserving logit key above the complement
// of the expert index, so keys are distinct and "greater" means larger logit, or
// equal logit and lower index; a key with r < k keys of its token above it is
// slot r.  Each wave takes 64 consecutive keys and one of rc shares of the keys
// they are compared with, so its lanes read the same LDS words together
// (broadcast reads); the shares meet through LDS atomics.  lr[j]: the logit of
// element tid + NT * j (loaded by the caller, early).  s_ck / s_rank: 12 * ne
// bytes of LDS.  Out: s_ids[8 * i + r] (expert of token i's slot r) and s_selk
// (its logit key).  Every thread of the workgroup calls it (two barriers inside;
// the caller's next barrier publishes the output).
template <int NT, int RK>
__device__ __forceinline__ void wg_route_rank(const float (&lr)[RK], int ne, int n_expert, int topk, int rc,
                                              uint64_t* s_ck, uint32_t* s_rank, int32_t* s_ids, uint32_t* s_selk) {
  const int tid = threadIdx.x, E = n_expert;
#pragma unroll
  for (int k = 0; k < RK; ++k) {
    const int q = tid + NT * k;
    if (q < ne) {
      const int e = q % E;
      s_ck[q] = ((uint64_t)route_key(lr[k]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
      s_rank[q] = 0;
    }
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  const int epp = NT / rc, c = tid / epp;
  for (int q0 = 0; q0 < ne; q0 += epp) {
    const int q = q0 + tid % epp;
    if (q < ne) {
      const int i = q / E;
      const uint64_t me = s_ck[q];
      const uint64_t* row = s_ck + i * E;
      const int f0 = c * E / rc, f1 = (c + 1) * E / rc;
      uint32_t above = 0;
#pragma unroll 8
      for (int f = f0; f < f1; ++f) above += row[f] > me ? 1u : 0u;
      if (rc == 1) s_rank[q] = above;
      else atomicAdd(&s_rank[q], above);
    }
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int k = 0; k < RK; ++k) {
    const int q = tid + NT * k;
    if (q < ne) {
      const int r = (int)s_rank[q];
      if (r < topk) {
        const int i = q / E;
        s_ids[8 * i + r] = q - i * E;
        s_selk[8 * i + r] = (uint32_t)(s_ck[q] >> 32);
      }
    }
  }
}

// The routing weights of the chunk from wg_route_rank's output, by one wave: lane
// p < t * topk (pair p = token p / topk, slot p % topk) gets its expert and weight
// (the router's softmax: exp of the logit minus the token's slot-0 logit, over
// their sum in slot order; every lane sums its token's row from s_ex, 64 floats of
// LDS, so no lane waits on another's chain).  Every lane of the wave calls it.
__device__ __forceinline__ void route_pair_weights(const int32_t* s_ids, const uint32_t* s_selk, float* s_ex, int t,
                                                   int topk, int lane, int& ep, float& wv) {
  const int ti = lane / topk, ki = lane - ti * topk;
  const bool pv = lane < t * topk;
  float ex = 0.0f;
  ep = 0;
  if (pv) {
    ep = s_ids[8 * ti + ki];
    ex = expf(route_val(s_selk[8 * ti + ki]) - route_val(s_selk[8 * ti]));
    s_ex[lane] = ex;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  float den = 0.0f;
  if (pv)
    for (int kk = 0; kk < topk; ++kk) den += s_ex[ti * topk + kk];
  wv = pv ? ex / den : 0.0f;
}

// ---------------------------------------------------------------------------
// routed-MoE helpers (direct route)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int clamp_id(int e, int64_t n_expert) {
  return e < 0 ? 0 : (e >= n_expert ? (int)n_expert - 1 : e);
}

// Which tokens of the chunk picked expert e = ids[slot]: bit i of mask, the slots
// of token i naming e in bits 8i.. of smask.  Returns false if an earlier slot
// already names e (that workgroup owns the expert).  Lane p reads pair p (one load
// per lane, t_real * topk <= 64); every lane of the wave must call it.
// ep: this lane's pair's expert (lane p = pair p; -1 past the pairs).
__device__ __forceinline__ bool expert_tokens_of(int ep, int slot, int t_real, int topk, int& e, uint32_t& mask,
                                                 uint64_t& smask) {
  const int p = threadIdx.x & 63, npairs = t_real * topk;
  e = __builtin_amdgcn_readlane(ep, slot);
  const uint64_t same = __ballot(p < npairs && ep == e);
  if (same & ((1ull << slot) - 1)) return false;
  mask = 0;
  smask = 0;
  for (int i = 0; i < t_real; ++i) {
    const uint64_t b = (same >> (i * topk)) & ((1ull << topk) - 1);
    smask |= b << (8 * i);
    if (b) mask |= 1u << i;
  }
  return true;
}
__device__ __forceinline__ bool expert_tokens(const int32_t* __restrict__ ids, int slot, int t_real, int topk,
                                              int64_t n_expert, int& e, uint32_t& mask, uint64_t& smask) {
  const int p = threadIdx.x & 63, npairs = t_real * topk;
  const int ep = p < npairs ? clamp_id(ids[p], n_expert) : -1;
  return expert_tokens_of(ep, slot, t_real, topk, e, mask, smask);
}

// index of the j-th set bit of m
__device__ __forceinline__ int nth_bit(uint32_t m, int j) {
  for (int s = 0; s < j; ++s) m &= m - 1;
  return __ffs(m) - 1;
}


// Reduce M values per lane over the lanes of an aligned group of L lanes
// (L a power of two <= 64, M <= L).  Afterwards value index i's group total sits
// in v[0] of lanes (i * L/M) .. (i * L/M + L/M - 1) of the group: each exchange
// step keeps the half of the values selected by the lane bit it pairs across.
// v_permlane{32,16}_swap(x, y) hands the lane whose bit S is clear (x_self,
// x_partner) and the lane whose bit S is set (y_partner, y_self), so with x the
// value the lower lane keeps and y the one the upper lane keeps, first + second
// is own + partner in every lane (no select; the sum is the same either order).
template <int S>
__device__ __forceinline__ float swap_sum(float x, float y) {
  static_assert(S == 16 || S == 32, "");
  uint32_t a = __float_as_uint(x), b = __float_as_uint(y);
  if constexpr (S == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

template <int M, int S>
__device__ __forceinline__ void reduce_level(float (&v)[M], int& m, int lane) {
  if constexpr (S == 16 || S == 32) {
    if (m > 1) {
#pragma unroll
      for (int i = 0; i < M / 2; ++i)
        if (i < m / 2) v[i] = swap_sum<S>(v[i], v[i + m / 2]);
      m >>= 1;
    } else {
      v[0] = swap_sum<S>(v[0], v[0]);
    }
    return;
  }
  if (m > 1) {
    const bool upper = (lane & S) != 0;
#pragma unroll
    for (int i = 0; i < M / 2; ++i) {
      if (i < m / 2) {
        const float keep = upper ? v[i + m / 2] : v[i];
        const float send = upper ? v[i] : v[i + m / 2];
        v[i] = keep + xchg<S>(send);
      }
    }
    m >>= 1;
  } else {
    v[0] += xchg<S>(v[0]);
  }
}

template <int M, int L>
__device__ __forceinline__ void group_reduce_multi(float (&v)[M], int lane) {
  static_assert(M <= L && L <= 64, "");
  int m = M;
  if constexpr (L >= 64) reduce_level<M, 32>(v, m, lane);
  if constexpr (L >= 32) reduce_level<M, 16>(v, m, lane);
  if constexpr (L >= 16) reduce_level<M, 8>(v, m, lane);
  if constexpr (L >= 8) reduce_level<M, 4>(v, m, lane);
  if constexpr (L >= 4) reduce_level<M, 2>(v, m, lane);
  if constexpr (L >= 2) reduce_level<M, 1>(v, m, lane);
}

// ---------------------------------------------------------------------------
// Direct-to-LDS loads (global_load_lds_dwordx4) and the waits that go with them.
// One wave-wide call moves 16 bytes per active lane from src (per lane) to
// lds_base + 16 * lane (lds_base uniform over the wave); no VGPRs hold the data.
// The load counts in the wave's vmcnt like any global load and its LDS write is
// done when the count says so.  __syncthreads() would drain every such load
// (its fence covers LDS writes), so a ring of DMA stages waits with
// wait_vm<N>() for its own stage and meets at lds_barrier(), whose fence covers
// only the wave's LDS instructions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 2 /* nt */);
}
// The same with the default cache policy, for rings whose stages share lines (the
// MXFP4 superblock windows) or whose bytes a later launch re-reads.  The dense
// matvec rings keep nt: with the default policy the headline kernel measured
// 7.39 -> 7.74 us.
__device__ __forceinline__ void lds_dma16_cached(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// Geometry of a per-wave LDS-DMA ring stage: 64 units of weight blocks (one
// segment of a row, or several whole rows of at most 64 units together), read
// as CPW 16-byte chunks per lane from the 16-byte boundary at or below its start.
template <int F> struct SegGeo {
  static constexpr int BYTES = 64 / Fmt<F>::UPB * Fmt<F>::BB;   // bytes of 64 units
  static constexpr int CPW = (BYTES + 15 + 1023) / 1024;         // 16-byte chunks per lane per stage
};

// wait until at most N global loads / stores of this wave are outstanding
// (gfx9 s_waitcnt: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8 left at max)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// a ring of S stages of CPL loads each: wait until the oldest stage has landed
// while k (<= S - 1) later stages stay in flight
template <int CPL, int S>
__device__ __forceinline__ void wait_tiles(int k) {
  if constexpr (S > 3) if (k >= 3) { wait_vm<3 * CPL>(); return; }
  if constexpr (S > 2) if (k >= 2) { wait_vm<2 * CPL>(); return; }
  if constexpr (S > 1) if (k >= 1) { wait_vm<CPL>(); return; }
  wait_vm<0>();
}

// workgroup barrier after this wave's LDS reads and writes (lgkmcnt(0)); global
// loads in flight, DMA or not, stay in flight
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace ftk
