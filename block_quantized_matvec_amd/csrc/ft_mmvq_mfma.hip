// ft_mmvq_mfma.hip -- Q-matvec for 2..8 tokens on the int8 matrix cores
// (v_mfma_i32_16x16x32_i8): every weight format (Q4_0, Q8_0, Q4_K, Q5_K, Q6_K,
// MXFP4, Q2_K, Q3_K, Q4_1, Q5_0, Q5_1) against Q8_1 activations (Q5_K adds the fifth bits to Q4_K's nibbles;
// Q6_K enters as q6 - 32 with one MFMA per 16-element scale group, and so do Q2_K's
// 2-bit codes and Q3_K's q - 4; MXFP4 as twice its E2M1 values with 2^(e-128) as
// the block scale, in 512-element chunks; Q4_1 / Q5_0 / Q5_1 as Q4_0 with their
// fifth bits and the offset m from a second MFMA against an all-ones operand).
//
// The int8-activation quantized matvec (FreeToken PR #136, Summary: the
// production ggml_mul_mat_vec_a8 kernel and its numerical tests): a block's
// integer dot product of weight and activation codes, then the fp32 scale
// combine.  MI355X design for more than one token:
//  * the tokens are rows of the MFMA A operand (up to 16; 2..8 here) and 16 weight
//    rows its columns, so one instruction takes a 32-element block of 16 rows
//    against every token: no activation codes are held in VGPRs per token and the
//    per-token cost is the scale combine only (the dot4 kernels keep every
//    token's codes in VGPRs and spill from 4 tokens on);
//  * a workgroup owns 16 rows split over K in KP parts, one wave each; a wave
//    streams 256-element chunks of its 16 rows and of the activation rows into
//    its own LDS slice with 16-byte loads (the next chunk in VGPRs while the
//    current one is computed) and reads its operands from there; no barrier
//    until the parts are summed, in a fixed order, through LDS;
//  * per block: D = sum over the block of weight code x activation code (int32,
//    exact); y += D * (d_w * d_x) (Q8_0, and Q4_0 whose codes enter as n - 8);
//    Q4_K: y += d_x * (d * sc_j * D - dmin * m_j * S) with S the activation code
//    sum of sub-block j, from a second MFMA against an all-ones operand.
#include <stdlib.h>

#include "ft_device.h"
#include "ft_internal.h"

namespace ftk {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int MV_MAXT = 8;
constexpr int MV_CE = 256;   // elements of a row per chunk (512 for MXFP4)

// elements CE of a row's chunk and its bytes CB; a row's chunk goes to an LDS slot of
// NPR 16-byte pieces.  Chunks of whole pieces (CB % 16 == 0; MXFP4's 17-byte blocks
// need 512-element chunks for that) sit at the slot's start; Q6_K's 210-, Q3_K's
// 110- and Q2_K's 84-byte chunks are copied from the 16-byte boundary below them,
// one piece more, and read at their byte offset in the slot.
// PAD adds a piece to a whole-piece slot whose stride would put the 16 rows' reads
// of one offset on a few LDS banks (192-byte slots: 4-way conflicts); the pad piece
// re-reads the chunk's last one.
template <int F_, int CB_, int PAD_ = 0> struct MvSlot {
  static constexpr int CB = CB_;
  static constexpr bool UNAL = CB % 16 != 0;
  static constexpr int NPR = UNAL ? (CB + 30) / 16 : CB / 16 + PAD_;
  static constexpr int SLOT = 16 * NPR;
};
template <int F, int CE_ = MV_CE> struct MvGeo;
template <int CE_> struct MvGeo<FT_Q4_0, CE_> : MvSlot<FT_Q4_0, 18 * 256 / 32> { static constexpr int CE = 256; };
template <int CE_> struct MvGeo<FT_Q8_0, CE_> : MvSlot<FT_Q8_0, 34 * 256 / 32> { static constexpr int CE = 256; };
template <int CE_> struct MvGeo<FT_Q4_K, CE_> : MvSlot<FT_Q4_K, 144> { static constexpr int CE = 256; };
template <int CE_> struct MvGeo<FT_Q5_K, CE_> : MvSlot<FT_Q5_K, 176> { static constexpr int CE = 256; };
template <int CE_> struct MvGeo<FT_Q6_K, CE_> : MvSlot<FT_Q6_K, 210> { static constexpr int CE = 256; };
template <int CE_> struct MvGeo<FT_MXFP4, CE_> : MvSlot<FT_MXFP4, 17 * 512 / 32> { static constexpr int CE = 512; };
template <int CE_> struct MvGeo<FT_Q2_K, CE_> : MvSlot<FT_Q2_K, 84> { static constexpr int CE = 256; };
template <int CE_> struct MvGeo<FT_Q4_1, CE_> : MvSlot<FT_Q4_1, 20 * 256 / 32> { static constexpr int CE = 256; };
template <int CE_> struct MvGeo<FT_Q5_0, CE_> : MvSlot<FT_Q5_0, 22 * 256 / 32> { static constexpr int CE = 256; };
template <int CE_> struct MvGeo<FT_Q5_1, CE_> : MvSlot<FT_Q5_1, 24 * 256 / 32, 1> { static constexpr int CE = 256; };
template <int CE_> struct MvGeo<FT_Q3_K, CE_> : MvSlot<FT_Q3_K, 110> { static constexpr int CE = 256; };

template <int F, int CE> struct MvRegs {
  static constexpr int ACB = 36 * CE / 32;                              // one token's Q8_1 chunk
  static constexpr int NW = (16 * MvGeo<F>::NPR + 63) / 64;            // 16-byte weight pieces per lane
  static constexpr int NA = (MV_MAXT * ACB / 16 + 63) / 64;           // activation pieces per lane
  u32x4 w[NW];
  u32x4 a[NA];
};

// 8 bytes at a 2- or 4-byte aligned LDS offset
__device__ __forceinline__ uint64_t lds_u64(const uint8_t* base, uint32_t off) {
  const uint32_t* d = (const uint32_t*)(base + (off & ~3u));
  const uint32_t s = off & 3u;
  const uint32_t d0 = d[0], d1 = d[1];
  if (s == 0) return (uint64_t)d0 | ((uint64_t)d1 << 32);
  const uint32_t d2 = d[2];
  return (uint64_t)__builtin_amdgcn_alignbyte(d1, d0, s) | ((uint64_t)__builtin_amdgcn_alignbyte(d2, d1, s) << 32);
}
__device__ __forceinline__ float lds_h2f(const uint8_t* base, uint32_t off) {
  return h2f(*(const uint16_t*)(base + off));
}

template <int F, int KP, int NR>
__global__ void __launch_bounds__(64 * KP)
mmvq_mfma_kernel(const uint8_t* __restrict__ W, int64_t n, int64_t k, int64_t row_bytes,
                 const uint8_t* __restrict__ xq, int64_t xrb, int t, float* __restrict__ y, int64_t ldy) {
  constexpr int CE = MvGeo<F>::CE;
  using R = MvRegs<F, CE>;
  using GE = MvGeo<F>;
  constexpr int CB = GE::CB, NPR = GE::NPR, SLOT = GE::SLOT, NWP = 16 * NPR, MV_ACB = R::ACB;
  constexpr int SLICE = 16 * SLOT + MV_MAXT * MV_ACB;
  constexpr int APT = MV_ACB / 16;   // activation pieces per token
  extern __shared__ u32x4 smem4[];
  const int lane = threadIdx.x & 63, wave = wave_id();
  uint8_t* wl = (uint8_t*)smem4 + wave * SLICE;   // this wave's 16 row slots
  uint8_t* al = wl + 16 * SLOT;                   // t activation rows x MV_ACB
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int nch = (int)(k / CE), c0 = wave * nch / KP, c1 = (wave + 1) * nch / KP;
  const int nap = APT * t;   // activation pieces per chunk

  // Every lane issues every load (pieces past the end, rows past n and chunks past
  // the part re-read valid bytes of the part that are never committed or used), so
  // that the loads in flight are the same on every path and the waits stay exact.
  // Re-reads stay inside the part: a neighbouring part's chunk read early would be
  // fetched from HBM twice.
  const int clast = c1 > c0 ? c1 - 1 : c0;
  auto fetch = [&](int c, R& r) {
    c = c < clast ? c : clast;
#pragma unroll
    for (int i = 0; i < R::NW; ++i) {
      int p = lane + 64 * i;
      p = p < NWP ? p : NWP - 1;
      const int row = p / NPR;
      int pc = p - row * NPR;
      const int64_t gr = row0 + row < n ? row0 + row : n - 1;
      int64_t b = gr * row_bytes + (int64_t)c * CB;
      if constexpr (!GE::UNAL && GE::SLOT > CB) pc = pc < CB / 16 ? pc : CB / 16 - 1;   // the pad piece
      if constexpr (GE::UNAL) {   // from the 16-byte boundary; pieces past the chunk re-read its last one
        const int npc = ((int)(b & 15) + CB + 15) >> 4;
        pc = pc < npc ? pc : npc - 1;
        b &= ~(int64_t)15;
      }
      r.w[i] = *(const u32x4*)(W + b + 16 * pc);
    }
#pragma unroll
    for (int i = 0; i < R::NA; ++i) {
      int p = lane + 64 * i;
      p = p < nap ? p : nap - 1;
      const int tok = p / APT, off = (p - tok * APT) * 16;
      r.a[i] = *(const u32x4*)(xq + (int64_t)tok * xrb + (int64_t)c * MV_ACB + off);
    }
  };
  auto commit = [&](const R& r) {
#pragma unroll
    for (int i = 0; i < R::NW; ++i) {
      const int p = lane + 64 * i;
      if (p < NWP) *(u32x4*)(wl + 16 * p) = r.w[i];
    }
#pragma unroll
    for (int i = 0; i < R::NA; ++i) {
      const int p = lane + 64 * i;
      if (p < nap) *(u32x4*)(al + 16 * p) = r.a[i];
    }
  };

  // Token i sits in A row 4*(i % 4) + i / 4, so that result row 4*kq + r (lane
  // group kq) is token kq + 4*r: with t tokens only r < ceil(t/4) carries results
  // and every lane group has its share (the scale combine runs ceil(t/4) times per
  // lane, not 4).
  // NR = ceil(t / 4) result rows per lane carry tokens (a template argument, so
  // the per-block combine has no branches); slot r of a lane holds token kq + 4r,
  // and a slot past t reads token 0's scale and adds it times zero.  Every LDS
  // read is unconditional, so the compiler can batch them ahead of the MFMAs.
  const int col = lane & 15, kq = lane >> 4;
  const int atok = (col >> 2) + 4 * (col & 3);   // the token of A row col
  const bool arow = atok < t;
  const uint32_t arow_off = (uint32_t)((arow ? atok : 0) * MV_ACB);
  bool sv[NR];
  uint32_t s_off[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    sv[r] = kq + 4 * r < t;
    s_off[r] = (uint32_t)((sv[r] ? kq + 4 * r : 0) * MV_ACB);
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const v4i zi = {0, 0, 0, 0};

  // byte offset of this lane's row chunk in its slot (Q6_K)
  const int64_t col_row = row0 + (lane & 15) < n ? row0 + (lane & 15) : n - 1;
  auto compute = [&](int c) {
    if constexpr (F == FT_Q4_K || F == FT_Q5_K) {
      constexpr int SBB = F == FT_Q5_K ? 176 : 144, QS = F == FT_Q5_K ? 48 : 16;   // superblock, qs offset
#pragma unroll
     for (int sbk = 0; sbk < CE / 256; ++sbk) {
      const u32x4 hd = *(const u32x4*)(wl + col * CB + SBB * sbk);
      // Q5_K: fifth bits of elements 8kq..8kq+7 of every sub-block (bit j of qh[l])
      uint64_t qh = 0;
      if constexpr (F == FT_Q5_K) qh = *(const uint64_t*)(wl + col * CB + SBB * sbk + 16 + 8 * kq);
      const float d = h2f(hd.x & 0xFFFFu), dmin = h2f(hd.x >> 16);
      uint32_t sc_lo, sc_hi, m_lo, m_hi;
      kq_unpack_scales(hd.y, hd.z, hd.w, sc_lo, sc_hi, m_lo, m_hi);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t sh = 8u * (uint32_t)(j & 3);
        const float dsc = d * (float)(((j < 4 ? sc_lo : sc_hi) >> sh) & 0xFFu);
        const float dmn = dmin * (float)(((j < 4 ? m_lo : m_hi) >> sh) & 0xFFu);
        const uint64_t q = *(const uint64_t*)(wl + col * CB + SBB * sbk + QS + 32 * (j >> 1) + 8 * kq);
        uint64_t b = (j & 1) ? (q >> 4) & 0x0F0F0F0F0F0F0F0Full : q & 0x0F0F0F0F0F0F0F0Full;
        if constexpr (F == FT_Q5_K) b |= ((qh >> j) & 0x0101010101010101ull) << 4;
        const uint64_t ar = lds_u64(al, arow_off + (uint32_t)(288 * sbk + 36 * j + 4 + 8 * kq));
        const uint64_t a = arow ? ar : 0ull;
        const v4i D = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)a, (long)b, zi, 0, 0, 0);
        const v4i S = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)a, (long)0x0101010101010101ll, zi, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const float dxr = lds_h2f(al, s_off[r] + (uint32_t)(288 * sbk + 36 * j));
          const float dx = sv[r] ? dxr : 0.0f;
          acc[r] = fmaf(dx, fmaf(dsc, (float)D[r], -dmn * (float)S[r]), acc[r]);
        }
      }
     }
    } else if constexpr (F == FT_Q6_K) {
      // Q6_K: ql[128] @0, qh[64] @128, int8 scales[16] @192, fp16 d @208; the
      // 32-element block j = 4g + r holds elements 128g + 32r + l, l = 0..31, whose
      // halves l < 16 and l >= 16 have their own scale (2j, 2j + 1): two MFMAs per
      // block, each with the other half's lanes (kq >= 2 or kq < 2) zeroed.  Codes
      // enter as q6 - 32 (int8).
      const uint32_t base = (uint32_t)(col * SLOT) + (uint32_t)((col_row * row_bytes + (int64_t)c * CB) & 15);
      const float d = lds_h2f(wl, base + 208);
      const uint64_t sc_a = lds_u64(wl, base + 192), sc_b = lds_u64(wl, base + 200);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int g = j >> 2, rr = j & 3;
        const uint64_t q = lds_u64(wl, base + (uint32_t)(64 * g + 32 * (rr & 1) + 8 * kq));
        const uint64_t h = lds_u64(wl, base + (uint32_t)(128 + 32 * g + 8 * kq));
        uint64_t x = ((q >> (4 * (rr >> 1))) & 0x0F0F0F0F0F0F0F0Full) | (((h >> (2 * rr)) & 0x0303030303030303ull) << 4);
        // x - 32 in every byte (x <= 63): no borrow crosses a byte once bit 7 is set
        x = ((x | 0x8080808080808080ull) - 0x2020202020202020ull) ^ 0x8080808080808080ull;
        const uint64_t blo = kq < 2 ? x : 0ull, bhi = kq < 2 ? 0ull : x;
        const uint64_t scw = j < 4 ? sc_a : sc_b;
        const float sl = (float)(int8_t)(uint8_t)(scw >> (16 * (j & 3))), sh = (float)(int8_t)(uint8_t)(scw >> (16 * (j & 3) + 8));
        const uint64_t ar = lds_u64(al, arow_off + (uint32_t)(36 * j + 4 + 8 * kq));
        const uint64_t a = arow ? ar : 0ull;
        const v4i Dl = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)a, (long)blo, zi, 0, 0, 0);
        const v4i Dh = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)a, (long)bhi, zi, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const float dxr = lds_h2f(al, s_off[r] + (uint32_t)(36 * j));
          const float dx = sv[r] ? dxr : 0.0f;
          acc[r] = fmaf(dx, d * fmaf(sl, (float)Dl[r], sh * (float)Dh[r]), acc[r]);
        }
      }
    } else if constexpr (F == FT_Q2_K || F == FT_Q3_K) {
      // Q2_K: scale|min bytes[16] @0, qs[64] @16, d @80, dmin @82.  Q3_K: hmask[32]
      // @0, qs[64] @32, 6-bit scales[12] @96, d @108.  The 32-element block
      // j = 4g + r holds elements 128g + 32r + l: bits 2r..2r+1 of qs[32g + l]
      // (Q3_K: bit 4g + r of hmask[l] is the third bit; codes enter as q - 4).
      // Its halves l < 16 and l >= 16 are sub-blocks 2j and 2j + 1 with their own
      // scales: two MFMAs per block with the other half's lanes zeroed, and for
      // Q2_K's mins two more against all-ones halves (the activation code sums).
      const uint32_t base = (uint32_t)(col * SLOT) + (uint32_t)((col_row * row_bytes + (int64_t)c * CB) & 15);
      constexpr uint32_t QS = F == FT_Q2_K ? 16 : 32;
      constexpr uint64_t ONES = 0x0101010101010101ull;
      const uint64_t olo = kq < 2 ? ONES : 0ull, ohi = kq < 2 ? 0ull : ONES;
      float d, dmin = 0.0f;
      uint64_t sc_a = 0, sc_b = 0, hm = 0;
      uint32_t s3[4] = {0u, 0u, 0u, 0u};
      if constexpr (F == FT_Q2_K) {
        d = lds_h2f(wl, base + 80);
        dmin = lds_h2f(wl, base + 82);
        sc_a = lds_u64(wl, base);
        sc_b = lds_u64(wl, base + 8);
      } else {
        d = lds_h2f(wl, base + 108);
        const uint64_t s01 = lds_u64(wl, base + 96);
        const uint32_t s0 = (uint32_t)s01, s1 = (uint32_t)(s01 >> 32);
        const uint32_t s2 = (uint32_t)lds_u64(wl, base + 104);
        // byte p of s3[q] = stored scale 4q + p: low nibbles of bytes 0-7 are scales
        // 0-7, their high nibbles 8-15; byte 8 + p holds the top bits of scales p,
        // 4 + p, 8 + p, 12 + p in bit pairs 0, 2, 4, 6
        s3[0] = (s0 & 0x0F0F0F0Fu) | ((s2 & 0x03030303u) << 4);
        s3[1] = (s1 & 0x0F0F0F0Fu) | (((s2 >> 2) & 0x03030303u) << 4);
        s3[2] = ((s0 >> 4) & 0x0F0F0F0Fu) | (((s2 >> 4) & 0x03030303u) << 4);
        s3[3] = ((s1 >> 4) & 0x0F0F0F0Fu) | (((s2 >> 6) & 0x03030303u) << 4);
        hm = lds_u64(wl, base + 8 * kq);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int g = j >> 2, rr = j & 3;
        const uint64_t q = lds_u64(wl, base + QS + (uint32_t)(32 * g + 8 * kq));
        uint64_t x = (q >> (2 * rr)) & 0x0303030303030303ull;
        if constexpr (F == FT_Q3_K) {
          x |= ((hm >> (4 * g + rr)) & ONES) << 2;
          // x - 4 in every byte (x <= 7): no borrow crosses a byte once bit 7 is set
          x = ((x | 0x8080808080808080ull) - 0x0404040404040404ull) ^ 0x8080808080808080ull;
        }
        const uint64_t blo = kq < 2 ? x : 0ull, bhi = kq < 2 ? 0ull : x;
        const uint64_t ar = lds_u64(al, arow_off + (uint32_t)(36 * j + 4 + 8 * kq));
        const uint64_t a = arow ? ar : 0ull;
        const v4i Dl = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)a, (long)blo, zi, 0, 0, 0);
        const v4i Dh = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)a, (long)bhi, zi, 0, 0, 0);
        if constexpr (F == FT_Q2_K) {
          const v4i Sl = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)a, (long)olo, zi, 0, 0, 0);
          const v4i Sh = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)a, (long)ohi, zi, 0, 0, 0);
          const uint32_t sm = (uint32_t)((j < 4 ? sc_a : sc_b) >> (16 * (j & 3)));   // bytes 2j, 2j + 1
          const float dl = d * (float)(sm & 15), ml = dmin * (float)((sm >> 4) & 15);
          const float dh = d * (float)((sm >> 8) & 15), mh = dmin * (float)((sm >> 12) & 15);
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            const float dxr = lds_h2f(al, s_off[r] + (uint32_t)(36 * j));
            const float dx = sv[r] ? dxr : 0.0f;
            const float w = fmaf(dl, (float)Dl[r], fmaf(dh, (float)Dh[r], -fmaf(ml, (float)Sl[r], mh * (float)Sh[r])));
            acc[r] = fmaf(dx, w, acc[r]);
          }
        } else {
          const uint32_t sp = s3[j >> 1] >> (16 * (j & 1));   // scales 2j, 2j + 1
          const float sl = (float)((int)(sp & 0xFFu) - 32), sh = (float)((int)((sp >> 8) & 0xFFu) - 32);
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            const float dxr = lds_h2f(al, s_off[r] + (uint32_t)(36 * j));
            const float dx = sv[r] ? dxr : 0.0f;
            acc[r] = fmaf(dx, d * fmaf(sl, (float)Dl[r], sh * (float)Dh[r]), acc[r]);
          }
        }
      }
    } else {
      constexpr int BB = F == FT_Q8_0 ? 34 : F == FT_MXFP4 ? 17 : F == FT_Q4_1 ? 20 : F == FT_Q5_0 ? 22
                       : F == FT_Q5_1 ? 24 : 18;
      // header bytes (scale, offset, fifth bits) before the codes
      constexpr int HB = F == FT_MXFP4 ? 1 : F == FT_Q4_1 ? 4 : F == FT_Q5_0 ? 6 : F == FT_Q5_1 ? 8 : 2;
      constexpr bool OFS = F == FT_Q4_1 || F == FT_Q5_1;   // w = d*q + m
#pragma unroll
      for (int blk = 0; blk < CE / 32; ++blk) {
        const uint32_t wb = (uint32_t)(col * SLOT + BB * blk);
        float dw;
        if constexpr (F == FT_MXFP4) dw = e8m0_half(wl[wb]);   // codes enter doubled: 2^(e-128)
        else dw = lds_h2f(wl, wb);
        uint64_t b;
        if constexpr (F == FT_Q8_0) {
          b = lds_u64(wl, wb + 2 + 8 * kq);
        } else if constexpr (F == FT_MXFP4) {
          // elements 8kq..8kq+7 as Q4_0's nibbles, each E2M1 code as twice its value
          const uint64_t q = lds_u64(wl, wb + HB + 8 * (kq & 1));
          const uint64_t nib = (q >> (4 * (kq >> 1))) & 0x0F0F0F0F0F0F0F0Full;
          b = (uint64_t)e2m1x2_bytes((uint32_t)nib) | ((uint64_t)e2m1x2_bytes((uint32_t)(nib >> 32)) << 32);
        } else if constexpr (F == FT_Q4_1 || F == FT_Q5_0 || F == FT_Q5_1) {
          // nibbles as Q4_0's; the fifth bits of elements 8kq..8kq+7 are byte kq of qh
          const uint64_t q = lds_u64(wl, wb + HB + 8 * (kq & 1));
          uint64_t x = (q >> (4 * (kq >> 1))) & 0x0F0F0F0F0F0F0F0Full;
          if constexpr (F != FT_Q4_1) {
            const uint32_t hb = wl[wb + HB - 4 + kq];
            x |= ((uint64_t)spread4(hb) | ((uint64_t)spread4(hb >> 4) << 32)) << 4;
          }
          if constexpr (F == FT_Q5_0)   // q - 16 as int8 (q <= 31)
            x = (x + 0x7070707070707070ull) ^ 0x8080808080808080ull;
          b = x;
        } else {
          // elements 8kq..8kq+7: low nibbles of bytes 0..7 (kq 0) or 8..15 (kq 1),
          // high nibbles of the same (kq 2, 3); as int8 n - 8
          const uint64_t q = lds_u64(wl, wb + 2 + 8 * (kq & 1));
          const uint64_t nib = (q >> (4 * (kq >> 1))) & 0x0F0F0F0F0F0F0F0Full;
          const uint32_t lo = ((uint32_t)nib + 0x78787878u) ^ 0x80808080u;
          const uint32_t hi = ((uint32_t)(nib >> 32) + 0x78787878u) ^ 0x80808080u;
          b = (uint64_t)lo | ((uint64_t)hi << 32);
        }
        const uint64_t ar = lds_u64(al, arow_off + (uint32_t)(36 * blk + 4 + 8 * kq));
        const uint64_t a = arow ? ar : 0ull;
        const v4i D = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)a, (long)b, zi, 0, 0, 0);
        if constexpr (OFS) {   // + m * (activation code sum), the sum from an all-ones operand
          const float m = lds_h2f(wl, wb + 2);
          const v4i S = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)a, (long)0x0101010101010101ll, zi, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            const float dxr = lds_h2f(al, s_off[r] + (uint32_t)(36 * blk));
            const float dx = sv[r] ? dxr : 0.0f;
            acc[r] = fmaf(dx, fmaf(dw, (float)D[r], m * (float)S[r]), acc[r]);
          }
        } else {
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            const float dxr = lds_h2f(al, s_off[r] + (uint32_t)(36 * blk));
            const float dx = sv[r] ? dxr : 0.0f;
            acc[r] = fmaf((float)D[r], dw * dx, acc[r]);
          }
        }
      }
    }
  };

  // one register buffer: chunk c + 1 is in flight while chunk c is computed
  R ra;
  fetch(c0, ra);
  for (int c = c0; c < c1; ++c) {
    commit(ra);
    fetch(c + 1, ra);
    // keep the loads ahead of the compute: the scheduler would otherwise sink
    // them to their use in the next commit (shorter live ranges, no overlap)
    __builtin_amdgcn_sched_barrier(0);
    compute(c);
  }

  // the KP parts, in order, through LDS (the slices are free now)
  __syncthreads();
  float* red = (float*)smem4;
  *(u32x4*)(red + (wave * 64 + lane) * 4) =
      u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]), __float_as_uint(acc[3])};
  __syncthreads();
  if (wave != 0) return;
  const int64_t row = row0 + col;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tok = kq + 4 * r;
    if (tok < t && row < n) {
      float s = red[lane * 4 + r];
      for (int q = 1; q < KP; ++q) s += red[(q * 64 + lane) * 4 + r];
      y[(int64_t)tok * ldy + row] = s;
    }
  }
}

template <int F, int KP>
static hipError_t launch_mfma_kp(const MmvqArgs& a, int64_t k, hipStream_t st) {
  constexpr int SLICE = 16 * MvGeo<F>::SLOT + MV_MAXT * MvRegs<F, MvGeo<F>::CE>::ACB;
  const dim3 grid((unsigned)((a.n + 15) / 16)), block(64 * KP);
  if (a.t <= 4)
    hipLaunchKernelGGL((mmvq_mfma_kernel<F, KP, 1>), grid, block, (size_t)KP * SLICE, st, (const uint8_t*)a.W, a.n,
                       k, (int64_t)a.row_bytes, (const uint8_t*)a.xq, (int64_t)a.xrow_bytes, a.t, a.y, a.ldy);
  else
    hipLaunchKernelGGL((mmvq_mfma_kernel<F, KP, 2>), grid, block, (size_t)KP * SLICE, st, (const uint8_t*)a.W, a.n,
                       k, (int64_t)a.row_bytes, (const uint8_t*)a.xq, (int64_t)a.xrow_bytes, a.t, a.y, a.ldy);
  return hipGetLastError();
}

// K parts per 16 rows: 8, or 2 when there are many rows and a row's 256-element
// chunk is at least 256 bytes (Q8_0: longer runs per row).  Measured on 14336 x
// 4096 at 8 tokens with 2 / 4 / 8 parts: Q8_0 16.5 / 18.3 / 19.3 us, Q4_K 13.3 /
// 12.3 / 11.9 us; 4096 x 14336 needs 8 (2 parts: 2-3x slower).  512-element chunks
// or a second register buffer cost more in occupancy than they gain in
// contiguity.
template <int F>
static hipError_t launch_mfma_f(const MmvqArgs& a, int64_t k, hipStream_t st) {
  const int64_t groups = (a.n + 15) / 16;
  const bool many = groups * 4 >= (int64_t)ftk_num_cus() * 8;
  if (many && MvGeo<F>::CB >= 256 && F == FT_Q8_0) return launch_mfma_kp<F, 2>(a, k, st);
  return launch_mfma_kp<F, 8>(a, k, st);
}

}  // namespace ftk

// 2..8 tokens, K a whole number of chunks, every weight format x Q8_1
static bool is_mmvq_mfma_format(int w) {
  return w == FT_Q4_0 || w == FT_Q8_0 || w == FT_Q4_K || w == FT_Q5_K || w == FT_Q6_K || w == FT_MXFP4 ||
         w == FT_Q2_K || w == FT_Q3_K || w == FT_Q4_1 || w == FT_Q5_0 || w == FT_Q5_1;
}

bool ftk_mmvq_mfma_ok(int w, int act, int64_t k, int t) {
  using namespace ftk;
  const int ce = w == FT_MXFP4 ? MvGeo<FT_MXFP4>::CE : MV_CE;
  return act == FT_Q8_1 && is_mmvq_mfma_format(w) &&
         k % ce == 0 && k > 0 && t >= 2 && t <= MV_MAXT;
}

hipError_t ftk_launch_mmvq_mfma(const MmvqArgs& a, int64_t k, hipStream_t st) {
  using namespace ftk;
  switch (a.w) {
    case FT_Q4_0: return launch_mfma_f<FT_Q4_0>(a, k, st);
    case FT_Q8_0: return launch_mfma_f<FT_Q8_0>(a, k, st);
    case FT_Q4_K: return launch_mfma_f<FT_Q4_K>(a, k, st);
    case FT_Q5_K: return launch_mfma_f<FT_Q5_K>(a, k, st);
    case FT_Q6_K: return launch_mfma_f<FT_Q6_K>(a, k, st);
    case FT_MXFP4: return launch_mfma_f<FT_MXFP4>(a, k, st);
    case FT_Q2_K: return launch_mfma_f<FT_Q2_K>(a, k, st);
    case FT_Q3_K: return launch_mfma_f<FT_Q3_K>(a, k, st);
    case FT_Q4_1: return launch_mfma_f<FT_Q4_1>(a, k, st);
    case FT_Q5_0: return launch_mfma_f<FT_Q5_0>(a, k, st);
    case FT_Q5_1: return launch_mfma_f<FT_Q5_1>(a, k, st);
    default: return hipErrorInvalidValue;
  }
}
