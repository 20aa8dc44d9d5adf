// ft_grouped.hip -- grouped keep-quant expert GEMM over expert-sorted pairs, on
// int8 MFMA.
//
// vllm.cpp PR #523 "grouped + non-grouped keep-quant expert GEMM" (What changed:
// the keep-quant op grouped over expert_ids, with a superblock integer dot core)
// and ds4 PR #656 (Summary: larger batches on expert-sorted tiles).
// y[p] = W[ids[p]] . xhat_row(p), p = token*topk + slot.  The token->expert sort
// (ft_moe.hip) gives each expert its contiguous list of pairs.
//
// Contraction on gfx950 (wave64, v_mfma_i32_16x16x32_i8):
//  * A workgroup owns (expert, 128 output rows; 64 for Q6_K); each of its four
//    waves owns 32 rows as two 16-row MFMA B operands that share every A-operand
//    read (16 rows for Q6_K, whose two MFMAs and two scales per group need the
//    registers), and every pair of the expert passes through it in tiles of 16
//    pairs (the A operand).  The expert's weight bytes are read from HBM once.
//  * Lane l of an MFMA holds weight row l%16 and the 8 codes 8(l/16)..8(l/16)+7 of
//    every 32-element group; the int32 result of one group is scaled by that
//    row's integer sub-block scale in the same lane (one v_mad_i32_i24 per output
//    and sub-block).  Q6_K's 16-element sub-blocks take two MFMAs per group whose
//    A operands are zero in the other half's lanes (those lanes read an all-zero
//    LDS tile).
//  * The K-quant min term sum_j m_j*B_j (B_j = sum of the activation codes of
//    sub-block j) and Q6_K's -32 offset term run on v_mfma_f32_16x16x16_f16 over
//    the 16-element code sums, which are exact in fp16 (|sum| <= 2032) and whose
//    products and sums are exact in fp32.
//  * MXFP4 runs on the block-scaled v_mfma_scale_f32_16x16x128_f8f6f4: the weights'
//    qs bytes are the FP4 B operand as stored and their E8M0 bytes the B scales;
//    the Q8_K codes enter as two exact FP8 halves x = 16*hi + lo (split once per
//    activation row beforehand), lo with scale 1 and hi with scale 2^4 chained in
//    one accumulator.  No E2M1 decode and no per-block scaling in the VALU.
//  * Per 256-element superblock the workgroup stages the activations of up to PT
//    pair tiles into LDS, in MFMA A-operand order, with the 16-element code sums
//    computed from the codes; each wave stages its rows' weight bytes into its own
//    LDS slots with 16-byte loads.  Both are fetched into VGPRs one superblock
//    ahead and published to LDS between two barriers.
//  * Workgroups are numbered so that all row tiles of one expert run on one XCD
//    (dispatch goes round-robin over the eight XCDs), so an expert's activation
//    rows are fetched into one L2.
// Rows never mix across pairs, so the order inside the sort cannot change any
// result.
#include <math.h>

#include "ft_device.h"
#include "ft_internal.h"

namespace ftk {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int GM_WAVES = 4;
constexpr int GM_THREADS = 64 * GM_WAVES;
// 16-row MFMA groups per wave (they share every A-operand read); Q6_K's two
// MFMAs and two scales per group need the registers of a second group, except in
// the fused gate/up form, whose two groups are the gate and up rows
template <int F, bool GLU> struct GRg { static constexpr int RG = (F == FT_Q6_K && !GLU) ? 1 : 2; };

// One 256-element superblock of a weight row: BYTES in HBM; SLOT bytes in LDS
// (room for a misaligned start; SLOT/16 odd keeps the 16 rows of an MFMA group on
// distinct LDS banks).
template <int F> struct GSb;
template <> struct GSb<FT_Q4_K> { static constexpr int BYTES = 144, SLOT = 144; static constexpr bool ALIGNED = true; };
template <> struct GSb<FT_Q5_K> { static constexpr int BYTES = 176, SLOT = 176; static constexpr bool ALIGNED = true; };
template <> struct GSb<FT_Q6_K> { static constexpr int BYTES = 210, SLOT = 240; static constexpr bool ALIGNED = false; };
template <> struct GSb<FT_MXFP4> { static constexpr int BYTES = 136, SLOT = 176; static constexpr bool ALIGNED = false; };

// LDS layout (bytes) for PT pair tiles: one superblock's buffer of BUF bytes, then
// the all-zero tile of the Q6_K half masks.
// MXFP4 tiles hold the FP8 halves instead: [PT][2 k-steps][lo, hi][2 16-byte
// halves][64 lanes] x 16 B, and need no code sums.
template <int F, int PT, int RG> struct GLds {
  static constexpr bool FP4 = F == FT_MXFP4;
  static constexpr int GSTR = 544;                       // bytes per 32-element group (512 + bank pad)
  static constexpr int TSTR = FP4 ? 8192 : 8 * GSTR;     // bytes per pair tile
  static constexpr int CODES = 0;                        // [PT][8 groups][64 lanes] x 8 B (+ pad)
  static constexpr int BSUM = CODES + PT * TSTR;         // [PT][64 lanes] x 4 fp16
  static constexpr int DX = BSUM + (FP4 ? 0 : PT * 512); // [PT][16 pairs] fp32
  static constexpr int WT = DX + PT * 64;                // [waves][16*RG rows][SLOT]
  static constexpr int BUF = WT + GM_WAVES * 16 * RG * GSb<F>::SLOT;
  static constexpr int ZTILE = BUF;                      // the zero tile
  static constexpr int TOTAL = ZTILE + (F == FT_Q6_K ? TSTR : 0);
};

// Weight operands of one 16-row group for one superblock, in one lane.
template <int F> struct GW {
  uint64_t b[8];    // int8 codes of the lane's 8 elements of each 32-element group
  int sc[8];        // integer sub-block scales (Q4_K/Q5_K)
  uint32_t scp[4];  // Q6_K: the 16 int8 sub-block scales, packed
  u32x4 fq[2];      // MXFP4: the raw qs bytes of block 4s + q (FP4 MFMA B operand), k-step s
  int e8[2];        // MXFP4: their E8M0 scale bytes
  v4h mb;           // f16 MFMA B operand of the min / offset term
  float d, dmin;
};

__device__ __forceinline__ uint64_t pk64(uint32_t lo, uint32_t hi) { return (uint64_t)lo | ((uint64_t)hi << 32); }

// Decode the lane's share of one superblock from its row slot (LDS).  o: byte
// offset of the superblock in the slot (0 for the 16-byte-aligned formats).
template <int F>
__device__ __forceinline__ void gw_decode(const uint8_t* sl, uint32_t o, int q, GW<F>& w) {
  if constexpr (F == FT_Q4_K || F == FT_Q5_K) {
    const u32x4 h = *(const u32x4*)sl;
    uint32_t sc_lo, sc_hi, m_lo, m_hi;
    kq_unpack_scales(h.y, h.z, h.w, sc_lo, sc_hi, m_lo, m_hi);
    w.d = h2f(h.x & 0xFFFFu);
    w.dmin = h2f(h.x >> 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w.sc[j] = (int)((sc_lo >> (8 * j)) & 0xFFu);
      w.sc[4 + j] = (int)((sc_hi >> (8 * j)) & 0xFFu);
    }
    // min operand: lane quarter q covers code sums 4q..4q+3 = sub-blocks 2q, 2q+1
    const uint32_t mm = ((q < 2) ? m_lo : m_hi) >> (16 * (q & 1));
    const _Float16 ma = (_Float16)(float)(mm & 0xFFu), mb = (_Float16)(float)((mm >> 8) & 0xFFu);
    w.mb = (v4h){ma, ma, mb, mb};
    uint32_t e0 = 0, e1 = 0;
    if constexpr (F == FT_Q5_K) {
      const u32x2 e = *(const u32x2*)(sl + 16 + 8 * q);
      e0 = e.x;
      e1 = e.y;
    }
    constexpr int QO = F == FT_Q4_K ? 16 : 48;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x2 v = *(const u32x2*)(sl + QO + 32 * c + 8 * q);
      uint32_t l0 = v.x & 0x0F0F0F0Fu, l1 = v.y & 0x0F0F0F0Fu;
      uint32_t h0 = (v.x >> 4) & 0x0F0F0F0Fu, h1 = (v.y >> 4) & 0x0F0F0F0Fu;
      if constexpr (F == FT_Q5_K) {
        l0 |= ((e0 >> (2 * c)) & 0x01010101u) << 4;
        l1 |= ((e1 >> (2 * c)) & 0x01010101u) << 4;
        h0 |= ((e0 >> (2 * c + 1)) & 0x01010101u) << 4;
        h1 |= ((e1 >> (2 * c + 1)) & 0x01010101u) << 4;
      }
      w.b[2 * c] = pk64(l0, l1);
      w.b[2 * c + 1] = pk64(h0, h1);
    }
  } else if constexpr (F == FT_Q6_K) {
    const Reader<const uint32_t*> rd{(const uint32_t*)sl};
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      uint32_t a[2], bq[2], hq[2];
      rd.template dwords<2>(o + 64 * g + 8 * q, a);        // groups r = 0 (low nibbles), 2 (high)
      rd.template dwords<2>(o + 64 * g + 32 + 8 * q, bq);  // groups r = 1, 3
      rd.template dwords<2>(o + 128 + 32 * g + 8 * q, hq); // top two bits of all four
      uint32_t c[4][2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        c[0][m] = (a[m] & 0x0F0F0F0Fu) | ((hq[m] << 4) & 0x30303030u);
        c[1][m] = (bq[m] & 0x0F0F0F0Fu) | ((hq[m] << 2) & 0x30303030u);
        c[2][m] = ((a[m] >> 4) & 0x0F0F0F0Fu) | (hq[m] & 0x30303030u);
        c[3][m] = ((bq[m] >> 4) & 0x0F0F0F0Fu) | ((hq[m] >> 2) & 0x30303030u);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) w.b[4 * g + r] = pk64(c[r][0], c[r][1]);
    }
    uint32_t s4[4];
    rd.template dwords<4>(o + 192, s4);
#pragma unroll
    for (int i = 0; i < 4; ++i) w.scp[i] = s4[i];   // int8 scales stay packed (register pressure)
    const uint32_t sq = q == 0 ? s4[0] : q == 1 ? s4[1] : q == 2 ? s4[2] : s4[3];
    w.mb = (v4h){(_Float16)(float)(int8_t)(sq & 0xFFu), (_Float16)(float)(int8_t)((sq >> 8) & 0xFFu),
                 (_Float16)(float)(int8_t)((sq >> 16) & 0xFFu), (_Float16)(float)(int8_t)(sq >> 24)};
    w.d = h2f(rd.u16(o + 208));
    w.dmin = 0.0f;
  } else {  // MXFP4: lane quarter q takes block 4s + q of k-step s (17 bytes: E8M0, qs[16])
    const Reader<const uint32_t*> rd{(const uint32_t*)sl};
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const uint32_t bo = o + 17 * (4 * st + q);
      uint32_t v[4];
      rd.template dwords<4>(bo + 1, v);
      w.fq[st] = (u32x4){v[0], v[1], v[2], v[3]};
      w.e8[st] = (int)rd.u8(bo);
    }
    w.d = 0.0f;
    w.dmin = 0.0f;
  }
}

// GLU: W is the gate bank and W2 the up bank of the same shape; a wave's two row
// groups are the gate and up rows of the same 16 outputs, and y receives
// h = silu(g) * u (g, u also written to g_tap / u_tap when those are non-null).
template <int F, int PT, bool GLU>
__global__ void __launch_bounds__(GM_THREADS)
grouped_mfma_kernel(const uint8_t* __restrict__ W, const uint8_t* __restrict__ W2, int64_t n, int64_t row_bytes,
                    int nsb, const uint8_t* __restrict__ xq, int64_t xrow_bytes, const uint8_t* __restrict__ xf8,
                    int x_per_pair, int topk,
                    const int32_t* __restrict__ offsets, const int32_t* __restrict__ pairs,
                    float* __restrict__ y, float* __restrict__ g_tap, float* __restrict__ u_tap,
                    int64_t row_tiles, int64_t total, int64_t per_xcd) {
  using SB = GSb<F>;
  constexpr int RG = GRg<F, GLU>::RG;
  using LY = GLds<F, PT, RG>;
  constexpr int NCH = SB::SLOT / 16;                   // 16-byte chunks per row slot
  static_assert(!GLU || RG == 2, "the fused gate/up form takes two row groups");
  constexpr int WROWS = 16 * RG;                       // weight rows per wave
  constexpr int OROWS = GLU ? 16 : WROWS;              // output rows per wave
  constexpr int NWI = (WROWS * NCH + 63) / 64;         // weight chunks per lane
  constexpr bool FP4 = F == FT_MXFP4;                  // block-scaled FP4 x FP8 MFMA path
  constexpr int CPP = FP4 ? 32 : 16;                   // 16-byte activation chunks per pair and superblock
  constexpr int NAI = (PT * 16 * CPP + GM_THREADS - 1) / GM_THREADS;   // activation chunks per thread
  constexpr bool MINT = !FP4;                          // has a code-sum term
  constexpr bool KQ = F == FT_Q4_K || F == FT_Q5_K;
  extern __shared__ u32x4 gsm[];
  uint8_t* L = (uint8_t*)gsm;

  // XCD-aware numbering: consecutive (expert, row tile) items on one XCD
  const int64_t bid = blockIdx.x;
  const int64_t item = (bid & 7) * per_xcd + (bid >> 3);
  if (item >= total) return;
  const int e = (int)(item / row_tiles);
  const int64_t tile = item % row_tiles;
  const int p0 = offsets[e], p1 = offsets[e + 1];
  if (p0 >= p1) return;

  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int q = lane >> 4, rl = lane & 15;
  const int64_t wrow0 = tile * (OROWS * GM_WAVES) + (int64_t)wave * OROWS;   // first output row of this wave
  const uint8_t* wexp = W + (int64_t)e * n * row_bytes;
  const uint8_t* wexp2 = GLU ? W2 + (int64_t)e * n * row_bytes : wexp;
  // weight slot r of this wave: its bank and output row
  auto slot_src = [&](int r) { return (GLU && r >= 16) ? wexp2 : wexp; };
  auto slot_row = [&](int r) { return wrow0 + (GLU ? (r & 15) : r); };
  const int wslot = LY::WT + wave * WROWS * SB::SLOT;   // this wave's weight rows in a buffer
  const v4f zf = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (F == FT_Q6_K) {   // published by the first barrier of the superblock loop
    for (int i = tid; i < LY::TSTR / 16; i += GM_THREADS) ((u32x4*)(L + LY::ZTILE))[i] = (u32x4){0u, 0u, 0u, 0u};
  }

  for (int g0 = p0; g0 < p1; g0 += PT * 16) {
    const int gm = min(PT * 16, p1 - g0);
    const int npt = (gm + 15) >> 4;

    // activation staging: item it = tid + GM_THREADS*i.  Codes: chunk su = it % 16 (16
    // codes) of pair slot it / 16.  MXFP4: it = 512m + 64r + 16qa + spl is the 16-byte
    // slot of lane (qa, spl) in region r of tile m, so a wave writes 1 KB contiguously.
    auto fp4_item = [&](int it, int& m, int& r, int& qa, int& spl) {
      m = it >> 9;
      r = (it >> 6) & 7;
      qa = (it >> 4) & 3;
      spl = it & 15;
    };
    const uint8_t* xr[NAI];
    const uint8_t* xr8[NAI];
    int xpi[NAI], xpv[NAI];
#pragma unroll
    for (int i = 0; i < NAI; ++i) {
      int pi = (tid + GM_THREADS * i) / CPP;
      if constexpr (FP4) {
        int m, r, qa, spl;
        fp4_item(tid + GM_THREADS * i, m, r, qa, spl);
        pi = 16 * m + spl;
      }
      xpi[i] = pi;
      xpv[i] = pairs[g0 + min(pi, gm - 1)];   // every pair index in flight at once
    }
#pragma unroll
    for (int i = 0; i < NAI; ++i) {
      const int64_t row = x_per_pair ? xpv[i] : xpv[i] / topk;
      const bool live = xpi[i] < gm;
      xr[i] = live ? xq + row * xrow_bytes : nullptr;
      xr8[i] = (FP4 && live) ? xf8 + row * (int64_t)nsb * 512 : nullptr;
    }
    // chunk of the item: codes: su; MXFP4: the FP8 chunk c = 16p + 2j + h of region r
    // (r = 4*st + 2*pp + bh) and lane quarter qa: j = 4st + 2bh + (qa>>1), h = qa & 1
    int sui[NAI];
#pragma unroll
    for (int i = 0; i < NAI; ++i) {
      if constexpr (FP4) {
        int m, r, qa, spl;
        fp4_item(tid + GM_THREADS * i, m, r, qa, spl);
        const int st = r >> 2, pp = (r >> 1) & 1, bh = r & 1;
        sui[i] = 16 * pp + 2 * (4 * st + 2 * bh + (qa >> 1)) + (qa & 1);
      } else {
        sui[i] = tid % CPP;
      }
    }
    const int su = tid % CPP;

    u32x4 pa[NAI];
    float pdx[NAI];
    u32x4 pw[NWI];
    // each weight chunk's row start in global memory (null: the chunk is idle)
    const uint8_t* wrs[NWI];
#pragma unroll
    for (int i = 0; i < NWI; ++i) {
      const int c = lane + 64 * i;
      const int r = c / NCH;
      const int64_t row = slot_row(r);
      wrs[i] = (r < WROWS && row < n) ? slot_src(r) + row * row_bytes : nullptr;
    }
    auto fetch = [&](int sb) {
#pragma unroll
      for (int i = 0; i < NAI; ++i) {
        pa[i] = (u32x4){0u, 0u, 0u, 0u};
        pdx[i] = 0.0f;
        if (xr[i]) {
          if constexpr (FP4) {
            pa[i] = *(const u32x4*)(xr8[i] + (int64_t)sb * 512 + 16 * sui[i]);
          } else {
            const uint32_t* src = (const uint32_t*)(xr[i] + (int64_t)sb * 292 + 4 + 16 * su);
            pa[i] = (u32x4){src[0], src[1], src[2], src[3]};
          }
          if (sui[i] == 0) pdx[i] = *(const float*)(xr[i] + (int64_t)sb * 292);
        }
      }
#pragma unroll
      for (int i = 0; i < NWI; ++i) {
        const int ch = (lane + 64 * i) % NCH;
        if (wrs[i]) {
          const uint8_t* sp = wrs[i] + (int64_t)sb * SB::BYTES;
          const int sh = SB::ALIGNED ? 0 : (int)((uintptr_t)sp & 15);
          const int nch = (sh + SB::BYTES + 15) >> 4;
          // plain loads: the line that straddles two superblocks is read again by the next step
          if (SB::ALIGNED || ch < nch) pw[i] = *((const u32x4*)(sp - sh) + ch);
        }
      }
    };
    auto commit = [&](uint8_t* B) {
#pragma unroll
      for (int i = 0; i < NAI; ++i) {
        const int it = tid + GM_THREADS * i;
        if (FP4 && it < PT * 16 * CPP) {   // uniform per wave
          // region r = (2st + pp, bh) of tile m: [k-step st][part pp][byte half bh][lane]
          int m, r, qa, spl;
          fp4_item(it, m, r, qa, spl);
          *(u32x4*)(B + LY::CODES + m * LY::TSTR + r * 1024 + (qa * 16 + spl) * 16) = pa[i];
          if (sui[i] == 0) ((float*)(B + LY::DX))[m * 16 + spl] = pdx[i];
        } else if (!FP4 && it < PT * 16 * CPP) {   // uniform per wave
          const int pi = it >> 4, m = pi >> 4, spl = pi & 15;
          const int j = su >> 1, qa = 2 * (su & 1);
          uint64_t* cd = (uint64_t*)(B + LY::CODES + m * LY::TSTR + j * LY::GSTR);
          cd[qa * 16 + spl] = pk64(pa[i].x, pa[i].y);
          cd[(qa + 1) * 16 + spl] = pk64(pa[i].z, pa[i].w);
          if constexpr (MINT) {
            // code sum of this 16-element group; the quad su&~3 .. su|3 holds the
            // four sums one A-operand slot needs, gathered into its first lane
            const int s0 = dot4(pa[i].x, 0x01010101u, dot4(pa[i].y, 0x01010101u,
                           dot4(pa[i].z, 0x01010101u, dot4(pa[i].w, 0x01010101u, 0))));
            const float f0 = (float)s0;
            const float f1 = xchg<1>(f0), f2 = xchg<2>(f0);
            const float f3 = xchg<2>(f1);
            if ((su & 3) == 0) {
              const v4h hv = {(_Float16)f0, (_Float16)f1, (_Float16)f2, (_Float16)f3};
              *(v4h*)(B + LY::BSUM + m * 512 + 8 * ((su >> 2) * 16 + spl)) = hv;
            }
          }
          if (su == 0) ((float*)(B + LY::DX))[m * 16 + spl] = pdx[i];
        }
      }
#pragma unroll
      for (int i = 0; i < NWI; ++i)
        if (wrs[i]) *(u32x4*)(B + wslot + 16 * (lane + 64 * i)) = pw[i];   // slot r, chunk ch: 16 * (r * NCH + ch)
    };

    v4f acc[PT][RG];
#pragma unroll
    for (int m = 0; m < PT; ++m)
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) acc[m][rg] = zf;

    fetch(0);
    for (int sb = 0; sb < nsb; ++sb) {
      __syncthreads();   // the previous superblock's LDS reads are done
      commit(L);
      if (sb + 1 < nsb) fetch(sb + 1);
      __syncthreads();
      uint8_t* cur = L;

      GW<F> w[RG];
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        const int r = rg * 16 + rl;
        uint32_t o = 0;
        if constexpr (!SB::ALIGNED)
          o = (uint32_t)((uintptr_t)(slot_src(r) + slot_row(r) * row_bytes + (int64_t)sb * SB::BYTES) & 15);
        gw_decode<F>(cur + wslot + r * SB::SLOT, o, q, w[rg]);
      }
      // the occupied pair tiles against the lane's decoded row groups (the helper
      // arrays stay in registers only when this code is written inline)
      const v4i zi = {0, 0, 0, 0};
    #pragma unroll
      for (int m = 0; m < PT; ++m) {
        if (FP4 && m < npt) {
          // two k-steps x (lo, hi) chained in one accumulator: the hi half carries
          // scale 2^4 (E8M0 131), the weights their block's E8M0 byte
          const uint8_t* ab = cur + LY::CODES + m * LY::TSTR + 16 * lane;
          const v4f dx4 = *(const v4f*)(cur + LY::DX + m * 64 + 16 * q);
          v4f dd[RG];
    #pragma unroll
          for (int rg = 0; rg < RG; ++rg) dd[rg] = zf;
    #pragma unroll
          for (int st = 0; st < 2; ++st) {
    #pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
              const u32x4 a0 = *(const u32x4*)(ab + (st * 2 + pp) * 2048);
              const u32x4 a1 = *(const u32x4*)(ab + (st * 2 + pp) * 2048 + 1024);
              const v8i av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    #pragma unroll
              for (int rg = 0; rg < RG; ++rg) {
                const v8i bw = {(int)w[rg].fq[st].x, (int)w[rg].fq[st].y, (int)w[rg].fq[st].z, (int)w[rg].fq[st].w,
                                0, 0, 0, 0};
                dd[rg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bw, dd[rg], 0, 4, 0, pp ? 131 : 127, 0,
                                                                          w[rg].e8[st]);
              }
            }
          }
    #pragma unroll
          for (int rg = 0; rg < RG; ++rg)
    #pragma unroll
            for (int r = 0; r < 4; ++r) acc[m][rg][r] = fmaf(dx4[r], dd[rg][r], acc[m][rg][r]);
        } else if (!FP4 && m < npt) {
          const uint8_t* ac = cur + LY::CODES + m * LY::TSTR + 8 * lane;
          // Q6_K: the low half of a 32-element group (quarters 0, 1) is one sub-block
          // and the high half the next; each of its two MFMAs reads zeros in the other
          // half's lanes (an all-zero LDS tile)
          const uint8_t* az = L + LY::ZTILE + 8 * lane;
          const uint8_t* a0p = (F == FT_Q6_K && q >= 2) ? az : ac;
          const uint8_t* a1p = (F == FT_Q6_K && q < 2) ? az : ac;
          v4i isc[RG];
          v4f ys[RG];
    #pragma unroll
          for (int rg = 0; rg < RG; ++rg) {
            isc[rg] = zi;
            ys[rg] = zf;
          }
    #pragma unroll
          for (int j = 0; j < 8; ++j) {
            const long a0 = *(const long*)(a0p + j * LY::GSTR);
            long a1 = 0;
            if constexpr (F == FT_Q6_K) a1 = *(const long*)(a1p + j * LY::GSTR);
    #pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
              const v4i dv = __builtin_amdgcn_mfma_i32_16x16x32_i8(a0, (long)w[rg].b[j], zi, 0, 0, 0);
              if constexpr (KQ) {
    #pragma unroll
                for (int r = 0; r < 4; ++r) isc[rg][r] += __mul24(dv[r], w[rg].sc[j]);
              } else if constexpr (F == FT_Q6_K) {
                const v4i dh = __builtin_amdgcn_mfma_i32_16x16x32_i8(a1, (long)w[rg].b[j], zi, 0, 0, 0);
                const int s0 = (int)(int8_t)((w[rg].scp[j >> 1] >> (16 * (j & 1))) & 0xFFu);
                const int s1 = (int)(int8_t)((w[rg].scp[j >> 1] >> (16 * (j & 1) + 8)) & 0xFFu);
    #pragma unroll
                for (int r = 0; r < 4; ++r) isc[rg][r] += __mul24(dv[r], s0) + __mul24(dh[r], s1);
              } else {
    #pragma unroll
                for (int r = 0; r < 4; ++r) ys[rg][r] += (float)dv[r];   // not reached (MXFP4 takes the FP4 path)
              }
            }
          }
          const v4f dx4 = *(const v4f*)(cur + LY::DX + m * 64 + 16 * q);
          if constexpr (F != FT_MXFP4) {
            const v4h ba = *(const v4h*)(cur + LY::BSUM + m * 512 + 8 * lane);
    #pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
              const v4f dm = __builtin_amdgcn_mfma_f32_16x16x16f16(ba, w[rg].mb, zf, 0, 0, 0);
    #pragma unroll
              for (int r = 0; r < 4; ++r) {
                float t;
                if constexpr (KQ) t = fmaf(-w[rg].dmin, dm[r], w[rg].d * (float)isc[rg][r]);
                else t = w[rg].d * fmaf(-32.0f, dm[r], (float)isc[rg][r]);
                acc[m][rg][r] = fmaf(dx4[r], t, acc[m][rg][r]);
              }
            }
          } else {
    #pragma unroll
            for (int rg = 0; rg < RG; ++rg)
    #pragma unroll
              for (int r = 0; r < 4; ++r) acc[m][rg][r] = fmaf(dx4[r], ys[rg][r], acc[m][rg][r]);
          }
        }
      }
    }

    // lane holds weight slots 16rg + rl for pairs 16m + 4q + r of the group
#pragma unroll
    for (int m = 0; m < PT; ++m) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pi = 16 * m + 4 * q + r;
        if (pi < gm) {
          const int64_t pr = pairs[g0 + pi];
          if constexpr (GLU) {
            const int64_t row = wrow0 + rl;
            if (row < n) {
              const float g = acc[m][0][r], u = acc[m][1][r];
              y[pr * n + row] = g / (1.0f + expf(-g)) * u;
              if (g_tap) g_tap[pr * n + row] = g;
              if (u_tap) u_tap[pr * n + row] = u;
            }
          } else {
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
              const int64_t row = wrow0 + 16 * rg + rl;
              if (row < n) y[pr * n + row] = acc[m][rg][r];
            }
          }
        }
      }
    }
  }
}

// 4 bytes per lane by direct-to-LDS load, default cache policy (the pairs' Q8_K d)
__device__ __forceinline__ void lds_dma4_cached(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 4, 0, 0);
}

// ---------------------------------------------------------------------------
// The K-quant kernel with every operand staged by direct-to-LDS loads.  Same
// contraction as above; what differs is the staging:
//  * two LDS stages, one barrier per superblock: superblock sb+1 of the weights
//    and activations is in flight (global_load_lds) while sb is computed, and no
//    VGPR holds staged data;
//  * each pair's Q8_K superblock lands as stored (codes, group sums, d) in a
//    304-byte slot from the 16-byte boundary at or below its start, so a lane
//    reads its A operand at the superblock's offset in the slot; the min / offset
//    term takes the format's 16-element group sums as stored (exact in fp16);
//    wave 0 also moves the pairs' d into a dense array;
//  * the occupied pair tiles of a pass run interleaved (one code path per tile
//    count), so the MFMAs of different tiles hide each other's latency.
// Two stages of 37 KB (Q5_K, 3 tiles) keep two workgroups per CU.
// ---------------------------------------------------------------------------
template <int F, int PT, int RG> struct GDLds {
  static constexpr int XS = 304;                                     // one 292-byte Q8_K superblock, 16-byte aligned down
  static constexpr int WT = 0;                                       // [waves][16*RG rows][SLOT]
  static constexpr int X = WT + GM_WAVES * 16 * RG * GSb<F>::SLOT;   // [PT*16 pairs][XS]
  static constexpr int DX = X + PT * 16 * XS;                        // [PT*16] fp32 d
  static constexpr int STAGE = DX + PT * 64;
  static constexpr int ZERO = 2 * STAGE;                             // Q6_K: 256 zero bytes (half masks)
  static constexpr int TOTAL = ZERO + (F == FT_Q6_K ? 256 : 0);
  static_assert(STAGE % 16 == 0, "");
};

template <int N> struct GIc { static constexpr int value = N; };

template <int F, int PT, bool GLU>
__global__ void __launch_bounds__(GM_THREADS) __attribute__((amdgpu_waves_per_eu(2)))
grouped_dma_kernel(const uint8_t* __restrict__ W, const uint8_t* __restrict__ W2, int64_t n, int64_t row_bytes,
                   int nsb, const uint8_t* __restrict__ xq, int64_t xrow_bytes, int x_per_pair, int topk,
                   const int32_t* __restrict__ offsets, const int32_t* __restrict__ pairs,
                   float* __restrict__ y, float* __restrict__ g_tap, float* __restrict__ u_tap,
                   int64_t row_tiles, int64_t total, int64_t per_xcd) {
  using SB = GSb<F>;
  constexpr int RG = GRg<F, GLU>::RG;
  using LY = GDLds<F, PT, RG>;
  constexpr int NCH = SB::SLOT / 16;                   // 16-byte chunks per weight slot
  static_assert(!GLU || RG == 2, "the fused gate/up form takes two row groups");
  static_assert(F == FT_Q4_K || F == FT_Q5_K || F == FT_Q6_K, "K-quant weights");
  constexpr int WROWS = 16 * RG;
  constexpr int OROWS = GLU ? 16 : WROWS;
  constexpr int NWI = (WROWS * NCH + 63) / 64;         // weight chunks per lane
  constexpr int XCH = LY::XS / 16;                     // 16-byte chunks per activation slot
  constexpr int NXI = (PT * 16 * XCH + GM_THREADS - 1) / GM_THREADS;   // activation chunks per lane
  constexpr bool KQ = F == FT_Q4_K || F == FT_Q5_K;
  extern __shared__ u32x4 gsm[];
  uint8_t* L = (uint8_t*)gsm;

  const int64_t bid = blockIdx.x;
  const int64_t item = (bid & 7) * per_xcd + (bid >> 3);
  if (item >= total) return;
  const int e = (int)(item / row_tiles);
  const int64_t tile = item % row_tiles;
  const int p0 = offsets[e], p1 = offsets[e + 1];
  if (p0 >= p1) return;

  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int q = lane >> 4, rl = lane & 15;
  const int64_t wrow0 = tile * (OROWS * GM_WAVES) + (int64_t)wave * OROWS;
  const uint8_t* wexp = W + (int64_t)e * n * row_bytes;
  const uint8_t* wexp2 = GLU ? W2 + (int64_t)e * n * row_bytes : wexp;
  auto slot_src = [&](int r) { return (GLU && r >= 16) ? wexp2 : wexp; };
  auto slot_row = [&](int r) { return wrow0 + (GLU ? (r & 15) : r); };
  const int wslot = LY::WT + wave * WROWS * SB::SLOT;
  const v4f zf = {0.0f, 0.0f, 0.0f, 0.0f};
  const v4i zi = {0, 0, 0, 0};
  if constexpr (F == FT_Q6_K) {   // published by the first barrier of the superblock loop
    if (tid < 16) ((u32x4*)(L + LY::ZERO))[tid] = (u32x4){0u, 0u, 0u, 0u};
  }
  // this lane's weight chunks: row start (null: idle)
  const uint8_t* wrs[NWI];
#pragma unroll
  for (int i = 0; i < NWI; ++i) {
    const int c = lane + 64 * i;
    const int r = c / NCH;
    const int64_t row = slot_row(r);
    wrs[i] = (r < WROWS && row < n) ? slot_src(r) + row * row_bytes : nullptr;
  }
  auto xrow_of = [&](int p) -> const uint8_t* {
    const int64_t row = x_per_pair ? pairs[p] : pairs[p] / topk;
    return xq + row * xrow_bytes;
  };

  for (int g0 = p0; g0 < p1; g0 += PT * 16) {
    const int gm = min(PT * 16, p1 - g0);
    const int npt = (gm + 15) >> 4;
    // activation chunks: instruction i of wave w moves items 64*(GM_WAVES*i + w) + lane,
    // item = pair * XCH + chunk, to X + 16 * item
    const uint8_t* xrs[NXI];   // pair row start + 16 * chunk (null: idle)
#pragma unroll
    for (int i = 0; i < NXI; ++i) {
      const int it = 64 * (GM_WAVES * i + wave) + lane;
      const int pi = it / XCH;
      xrs[i] = (it < PT * 16 * XCH && pi < gm) ? xrow_of(g0 + pi) + 16 * (it - pi * XCH) : nullptr;
    }
    // wave 0: pair `lane`'s row, for its d
    const uint8_t* drs = (wave == 0 && lane < gm) ? xrow_of(g0 + lane) : nullptr;
    // the low address bits of the lane's own pair row in each tile (its superblock's offset in the slot)
    uint32_t xlo[PT];
#pragma unroll
    for (int m = 0; m < PT; ++m) {
      const int pi = 16 * m + rl;
      xlo[m] = pi < gm ? (uint32_t)(uintptr_t)xrow_of(g0 + pi) : 0u;
    }

    auto issue = [&](int sb, int s) {
      uint8_t* B = L + s * LY::STAGE;
#pragma unroll
      for (int i = 0; i < NWI; ++i) {
        const int ch = (lane + 64 * i) % NCH;
        if (wrs[i]) {
          const uint8_t* sp = wrs[i] + (int64_t)sb * SB::BYTES;
          const int sh = SB::ALIGNED ? 0 : (int)((uintptr_t)sp & 15);
          // chunks that overlap the superblock (16-byte aligned: never past the buffer's last line)
          if (SB::ALIGNED || ch < ((sh + SB::BYTES + 15) >> 4)) lds_dma16_cached(sp - sh + 16 * ch, B + wslot + 1024 * i);
        }
      }
#pragma unroll
      for (int i = 0; i < NXI; ++i) {
        if (xrs[i]) {
          const uint8_t* sp = xrs[i] + (int64_t)sb * 292;
          lds_dma16_cached(sp - ((uintptr_t)sp & 15), B + LY::X + 1024 * (GM_WAVES * i + wave));
        }
      }
      if (drs) lds_dma4_cached(drs + (int64_t)sb * 292, B + LY::DX);
    };

    v4f acc[PT][RG];
#pragma unroll
    for (int m = 0; m < PT; ++m)
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) acc[m][rg] = zf;

    issue(0, 0);
    for (int sb = 0; sb < nsb; ++sb) {
      wait_vm<0>();    // this wave's loads of superblock sb have landed
      lds_barrier();   // everyone's have; everyone is done with superblock sb-1's stage
      if (sb + 1 < nsb) issue(sb + 1, (sb + 1) & 1);
      const uint8_t* B = L + (sb & 1) * LY::STAGE;

      GW<F> w[RG];
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        const int r = rg * 16 + rl;
        uint32_t o = 0;
        if constexpr (!SB::ALIGNED)
          o = (uint32_t)((uintptr_t)(slot_src(r) + slot_row(r) * row_bytes + (int64_t)sb * SB::BYTES) & 15);
        gw_decode<F>(B + wslot + r * SB::SLOT, o, q, w[rg]);
      }

      // tiles M0 .. M0+NT-1, interleaved
      auto tiles = [&](auto m0c, auto ntc) {
        constexpr int M0 = decltype(m0c)::value, NT = decltype(ntc)::value;
        const uint8_t* ap[NT];   // the lane's codes (group 0, quarter q) in tile M0 + m
#pragma unroll
        for (int m = 0; m < NT; ++m)
          ap[m] = B + LY::X + LY::XS * (16 * (M0 + m) + rl) + ((xlo[M0 + m] + 4u * (uint32_t)sb) & 15u) + 4 + 8 * q;
        v4i isc[NT][RG];
#pragma unroll
        for (int m = 0; m < NT; ++m)
#pragma unroll
          for (int rg = 0; rg < RG; ++rg) isc[m][rg] = zi;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // every MFMA of the group first, then the integer scale step of each
          v4i dv[NT][RG], dh[NT][RG];
#pragma unroll
          for (int m = 0; m < NT; ++m) {
            const uint32_t* cp = (const uint32_t*)(ap[m] + 32 * j);
            long a0, a1 = 0;
            if constexpr (F == FT_Q6_K) {
              // the low half of a 32-element group (quarters 0, 1) is one sub-block and
              // the high half the next; each MFMA reads zeros in the other half's lanes
              const uint32_t* zp = (const uint32_t*)(L + LY::ZERO);
              const uint32_t* c0 = q >= 2 ? zp : cp;
              const uint32_t* c1 = q < 2 ? zp : cp;
              a0 = (long)pk64(c0[0], c0[1]);
              a1 = (long)pk64(c1[0], c1[1]);
            } else {
              a0 = (long)pk64(cp[0], cp[1]);
            }
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
              dv[m][rg] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a0, (long)w[rg].b[j], zi, 0, 0, 0);
              if constexpr (F == FT_Q6_K) dh[m][rg] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a1, (long)w[rg].b[j], zi, 0, 0, 0);
            }
          }
#pragma unroll
          for (int m = 0; m < NT; ++m) {
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
              if constexpr (KQ) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  isc[m][rg][r] += __mul24(dv[m][rg][r], w[rg].sc[j]);
                  // one multiply-add per product: keep the compiler from regrouping the
                  // chain into separate multiplies and three-way adds
                  asm("" : "+v"(isc[m][rg][r]));
                }
              } else {
                const int s0 = (int)(int8_t)((w[rg].scp[j >> 1] >> (16 * (j & 1))) & 0xFFu);
                const int s1 = (int)(int8_t)((w[rg].scp[j >> 1] >> (16 * (j & 1) + 8)) & 0xFFu);
#pragma unroll
                for (int r = 0; r < 4; ++r) isc[m][rg][r] += __mul24(dv[m][rg][r], s0) + __mul24(dh[m][rg][r], s1);
              }
            }
          }
        }
#pragma unroll
        for (int m = 0; m < NT; ++m) {
          // the lane's four 16-element group sums (int16 as stored, exact in fp16)
          const uint32_t* sp = (const uint32_t*)(ap[m] + 256);
          const uint32_t s01 = sp[0], s23 = sp[1];
          const v4h ba = {(_Float16)(int16_t)(s01 & 0xFFFFu), (_Float16)(int16_t)(s01 >> 16),
                          (_Float16)(int16_t)(s23 & 0xFFFFu), (_Float16)(int16_t)(s23 >> 16)};
          const v4f dx4 = *(const v4f*)(B + LY::DX + (M0 + m) * 64 + 16 * q);
#pragma unroll
          for (int rg = 0; rg < RG; ++rg) {
            const v4f dm = __builtin_amdgcn_mfma_f32_16x16x16f16(ba, w[rg].mb, zf, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float t;
              if constexpr (KQ) t = fmaf(-w[rg].dmin, dm[r], w[rg].d * (float)isc[m][rg][r]);
              else t = w[rg].d * fmaf(-32.0f, dm[r], (float)isc[m][rg][r]);
              acc[M0 + m][rg][r] = fmaf(dx4[r], t, acc[M0 + m][rg][r]);
            }
          }
        }
      };
      if constexpr (F == FT_Q6_K) {
        // two MFMAs and two scales per group: one tile at a time (registers)
        tiles(GIc<0>{}, GIc<1>{});
        if constexpr (PT >= 2) if (npt >= 2) tiles(GIc<1>{}, GIc<1>{});
        if constexpr (PT >= 3) if (npt >= 3) tiles(GIc<2>{}, GIc<1>{});
        if constexpr (PT >= 4) if (npt >= 4) tiles(GIc<3>{}, GIc<1>{});
      } else {
        if constexpr (PT >= 4) { if (npt >= 4) { tiles(GIc<0>{}, GIc<4>{}); continue; } }
        if constexpr (PT >= 3) { if (npt >= 3) { tiles(GIc<0>{}, GIc<3>{}); continue; } }
        if constexpr (PT >= 2) { if (npt >= 2) { tiles(GIc<0>{}, GIc<2>{}); continue; } }
        tiles(GIc<0>{}, GIc<1>{});
      }
    }

    // lane holds weight slots 16rg + rl for pairs 16m + 4q + r of the group
#pragma unroll
    for (int m = 0; m < PT; ++m) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pi = 16 * m + 4 * q + r;
        if (pi < gm) {
          const int64_t pr = pairs[g0 + pi];
          if constexpr (GLU) {
            const int64_t row = wrow0 + rl;
            if (row < n) {
              const float g = acc[m][0][r], u = acc[m][1][r];
              y[pr * n + row] = g / (1.0f + expf(-g)) * u;
              if (g_tap) g_tap[pr * n + row] = g;
              if (u_tap) u_tap[pr * n + row] = u;
            }
          } else {
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
              const int64_t row = wrow0 + 16 * rg + rl;
              if (row < n) y[pr * n + row] = acc[m][rg][r];
            }
          }
        }
      }
    }
    // the next pass overwrites both stages: everyone is done with the last one
    lds_barrier();
  }
}

template <int F, int PT, bool GLU>
static hipError_t launch_gd(const GroupedArgs& a, hipStream_t st) {
  constexpr int RG = GRg<F, GLU>::RG;
  const int rows = (GLU ? 16 : 16 * RG) * GM_WAVES;
  const int64_t row_tiles = (a.n + rows - 1) / rows;
  const int64_t total = row_tiles * a.n_expert;
  const int64_t per = (total + 7) / 8;
  const int64_t row_bytes = a.k / 256 * GSb<F>::BYTES;
  constexpr size_t lds = (size_t)GDLds<F, PT, RG>::TOTAL;
  static const bool attr = hipFuncSetAttribute((const void*)grouped_dma_kernel<F, PT, GLU>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess;
  if (!attr) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((grouped_dma_kernel<F, PT, GLU>), dim3((unsigned)(per * 8)), dim3(GM_THREADS), lds, st,
                     (const uint8_t*)a.W, (const uint8_t*)a.W2, a.n, row_bytes, (int)(a.k / 256),
                     (const uint8_t*)a.xq, (int64_t)(a.k / 256 * 292), a.x_per_pair, a.topk, a.offsets, a.pairs,
                     a.y, a.g_tap, a.u_tap, row_tiles, total, per);
  return hipGetLastError();
}

template <int F, int PT, bool GLU>
static hipError_t launch_gm(const GroupedArgs& a, hipStream_t st) {
  constexpr int RG = GRg<F, GLU>::RG;
  const int rows = (GLU ? 16 : 16 * RG) * GM_WAVES;
  const int64_t row_tiles = (a.n + rows - 1) / rows;
  const int64_t total = row_tiles * a.n_expert;
  const int64_t per = (total + 7) / 8;
  const int64_t row_bytes = a.k / 256 * GSb<F>::BYTES;
  const size_t lds = (size_t)GLds<F, PT, RG>::TOTAL;
  hipLaunchKernelGGL((grouped_mfma_kernel<F, PT, GLU>), dim3((unsigned)(per * 8)), dim3(GM_THREADS), lds, st,
                     (const uint8_t*)a.W, (const uint8_t*)a.W2, a.n, row_bytes, (int)(a.k / 256),
                     (const uint8_t*)a.xq, (int64_t)(a.k / 256 * 292), (const uint8_t*)a.xf8, a.x_per_pair, a.topk,
                     a.offsets, a.pairs,
                     a.y, a.g_tap, a.u_tap, row_tiles, total, per);
  return hipGetLastError();
}



// The DMA-staged kernel for Q4_K / Q5_K up to 3 pair tiles, where two of its
// workgroups fit a CU without spills; with its weight and activation loads on the
// default cache policy (the 136-176-byte superblock windows of a row share
// lines) it beats the register-staged kernel: Q5_K 1536x4096 gate/up at 512
// tokens 224 -> 207-208 us, down 228 -> 220-221 us, the K-quant tile layer 600 ->
// 577-579 us.  Q6_K stays on the register-staged kernel (down +2-4% on DMA).
template <int F, bool GLU, int PT>
static hipError_t launch_g(const GroupedArgs& a, hipStream_t st) {
  if constexpr (F == FT_Q4_K || F == FT_Q5_K) {
    if constexpr (PT <= 3) return launch_gd<F, PT, GLU>(a, st);
    else return launch_gm<F, PT, GLU>(a, st);
  } else {
    return launch_gm<F, PT, GLU>(a, st);
  }
}

// Pair tiles held per pass: room for an expert 2.5 standard deviations above the
// mean pairs per expert of this batch (uniform routing gives a near-binomial
// spread); a larger group takes a second pass over its weights.
template <int F, bool GLU>
static hipError_t grouped_f(const GroupedArgs& a, hipStream_t st) {
  const double avg = (double)a.t * a.topk / (double)a.n_expert;
  const double hi = avg + 2.5 * sqrt(avg);
  if (hi <= 16.0) return launch_g<F, GLU, 1>(a, st);
  if (hi <= 32.0) return launch_g<F, GLU, 2>(a, st);
  if (hi <= 48.0) return launch_g<F, GLU, 3>(a, st);
  return launch_g<F, GLU, 4>(a, st);
}

}  // namespace ftk

using namespace ftk;

hipError_t ftk_launch_grouped(const GroupedArgs& a, hipStream_t st) {
  if (a.act != FT_Q8_K || a.k % 256) return hipErrorInvalidValue;
  if (a.w == FT_MXFP4 && !a.xf8) return hipErrorInvalidValue;   // needs the FP8 halves
  if (a.W2) {   // fused gate/up + SwiGLU
    switch (a.w) {
      case FT_Q4_K: return grouped_f<FT_Q4_K, true>(a, st);
      case FT_Q5_K: return grouped_f<FT_Q5_K, true>(a, st);
      case FT_Q6_K: return grouped_f<FT_Q6_K, true>(a, st);
      case FT_MXFP4: return grouped_f<FT_MXFP4, true>(a, st);
    }
    return hipErrorInvalidValue;
  }
  switch (a.w) {
    case FT_Q4_K: return grouped_f<FT_Q4_K, false>(a, st);
    case FT_Q5_K: return grouped_f<FT_Q5_K, false>(a, st);
    case FT_Q6_K: return grouped_f<FT_Q6_K, false>(a, st);
    case FT_MXFP4: return grouped_f<FT_MXFP4, false>(a, st);
  }
  return hipErrorInvalidValue;
}
