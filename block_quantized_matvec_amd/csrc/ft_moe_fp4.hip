// ft_moe_fp4.hip -- direct-route MXFP4 expert kernels (gate/up + SwiGLU, down) on
// the block-scaled FP4 matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// ds4 PR #656 "Add ROCm MXFP4 routed expert kernels" (Summary): resident MXFP4 x
// Q8_K routed gate/up and down kernels with SwiGLU between them, and small batches
// sent through direct kernels rather than partly filled expert-sorted tiles.
// MI355X design:
//  * the tokens of a chunk (up to 8) are rows of the MFMA A operand and 16 weight
//    rows of one expert its columns; an MXFP4 block's 16 code bytes are one lane's
//    FP4 B operand as stored and its E8M0 byte that lane's B scale, so no E2M1
//    decode and no per-block scaling runs on the VALU;
//  * a Q8_K code x is not an FP8 value, so the activations enter as two exact
//    E4M3 halves x = 16*hi + lo (hi = x >> 4 in [-8, 7], lo = x & 15), chained in
//    one accumulator with A scales 2^0 and 2^4; per 256-element superblock the
//    four MFMAs (two k-steps x lo, hi) start from zero and the result is scaled by
//    the token's Q8_K scale;
//  * a workgroup of 8 waves owns 16-row groups of one expert, each split over K in
//    KQ parts (summed in a fixed order through LDS); odd parts walk K downwards so
//    that the cache line two parts share is fetched once;
//  * each lane takes its own block per k-step as five dwords (E8M0 byte + 16 code
//    bytes at a 1..4 byte offset): in gate/up (K a multiple of 512) from the
//    wave's LDS ring, filled by 16-byte global_load_lds over whole row pieces,
//    else straight from global memory one superblock ahead;
//  * the workgroup quantizes its activation rows to Q8_K itself (the arithmetic of
//    ft_quantize_act) and keeps them in LDS as the FP8 halves in the operand's
//    nibble order, with the Q8_K scale of every (token, superblock).
// The workgroup of the first slot naming an expert owns it and applies it to every
// token of the chunk that picked it.
#include <math.h>
#include <stdlib.h>

#include "ft_device.h"
#include "ft_internal.h"

namespace ftk {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int MF_WAVES = 8;
constexpr int MF_THREADS = 64 * MF_WAVES;
constexpr int MF_MAXT = 8;      // tokens per launch (A rows in use)

// Byte-wise table lookup of 4-bit indices (one per byte) in a 16-byte table t0..t3.
__device__ __forceinline__ uint32_t lut16(uint32_t n, uint32_t t0, uint32_t t1, uint32_t t2, uint32_t t3) {
  const uint32_t i = n & 0x07070707u;
  const uint32_t a = __builtin_amdgcn_perm(t1, t0, i);
  const uint32_t b = __builtin_amdgcn_perm(t3, t2, i);
  const uint32_t sel = ((n >> 1) & 0x04040404u) | 0x03020100u;   // byte k of a, or of b if index >= 8
  return __builtin_amdgcn_perm(b, a, sel);
}

// Four int8 codes -> their E4M3 (OCP) halves: lo = x & 15 (0..15), hi = x >> 4
// (two's-complement nibble: 0..7, then -8..-1).  1.0 is 0x38; every value is exact.
__device__ __forceinline__ void fp8_halves(uint32_t c, uint32_t& lo, uint32_t& hi) {
  lo = lut16(c & 0x0F0F0F0Fu, 0x44403800u, 0x4E4C4A48u, 0x53525150u, 0x57565554u);
  hi = lut16((c >> 4) & 0x0F0F0F0Fu, 0x44403800u, 0x4E4C4A48u, 0xCACCCED0u, 0xB8C0C4C8u);
}

// LDS activation image of one token: the lo halves of its K codes, then the hi
// halves (2K bytes), plus dx[superblock][16 tokens] fp32.  Within each 32-element
// block the codes are in the FP4 operand's nibble order: an MXFP4 block stores
// element e < 16 in the low nibble and e + 16 in the high nibble of byte e, and the
// MFMA takes nibble n (byte n/2, low first) as k-position n, so position n holds
// element n/2 + 16*(n & 1).
// Lane l16 holds elements 16*l16 .. 16*l16+15 of superblock sb (block l16/2, half
// h = l16&1) and writes positions 16h .. 16h+15 of that block: its own first (h=0)
// or the partner lane's second (h=1) eight codes interleaved with the partner's
// first or its own second eight.  Both lanes of a pair must call it.
__device__ __forceinline__ void stage_codes(const uint32_t (&w)[4], uint8_t* arow, int64_t k, int sb, int l16) {
  uint32_t pw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) pw[j] = (uint32_t)__float_as_int(xchg<1>(__int_as_float((int)w[j])));
  const bool h = l16 & 1;
  const uint32_t a0 = h ? pw[2] : w[0], a1 = h ? pw[3] : w[1];   // elements 8h .. 8h+7
  const uint32_t b0 = h ? w[2] : pw[0], b1 = h ? w[3] : pw[1];   // elements 16+8h .. 16+8h+7
  const uint32_t c[4] = {__builtin_amdgcn_perm(b0, a0, 0x05010400u), __builtin_amdgcn_perm(b0, a0, 0x07030602u),
                         __builtin_amdgcn_perm(b1, a1, 0x05010400u), __builtin_amdgcn_perm(b1, a1, 0x07030602u)};
  uint32_t lo[4], hi[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) fp8_halves(c[j], lo[j], hi[j]);
  *(u32x4*)(arow + 256 * sb + 16 * l16) = u32x4{lo[0], lo[1], lo[2], lo[3]};
  *(u32x4*)(arow + k + 256 * sb + 16 * l16) = u32x4{hi[0], hi[1], hi[2], hi[3]};
}

// One lane's MXFP4 block for k-step s: the 17 bytes at 68*s + 17*b of its row
// (b = lane >> 4) lie in the five dwords from dword 17*s + 4*b, at byte offset b.
struct Fp4Blk {
  uint32_t d[5];
};
__device__ __forceinline__ void fp4_fetch(const uint32_t* __restrict__ rowd, int s, int b, Fp4Blk& f) {
  const uint32_t* p = rowd + 17 * s + 4 * b;
#pragma unroll
  for (int i = 0; i < 5; ++i) f.d[i] = p[i];
}
// -> B operand (16 code bytes) and E8M0 scale byte
__device__ __forceinline__ v8i fp4_operand(const Fp4Blk& f, int b, int& e8) {
  const uint32_t sh = 8u * (uint32_t)(b + 1);   // 8..32 bits
  v8i o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = (int)(uint32_t)((((uint64_t)f.d[j + 1] << 32) | f.d[j]) >> sh);
  o[4] = o[5] = o[6] = o[7] = 0;
  e8 = (int)((f.d[0] >> (8 * b)) & 0xFFu);
  return o;
}

// The first superblock's blocks of a wave's rows (issued before the activation
// staging so that their latency overlaps it; unconditional, so that nothing
// waits for them early: a wave with no superblocks reads a valid one, unused).
template <int NM>
__device__ __forceinline__ void fp4_first(const uint32_t* const (&rowd)[NM], int sbf, int nsb, Fp4Blk (&nx)[NM][2]) {
  const int b = (threadIdx.x & 63) >> 4;
  sbf = sbf < 0 ? 0 : (sbf < nsb ? sbf : nsb - 1);
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    fp4_fetch(rowd[m], 2 * sbf, b, nx[m][0]);
    fp4_fetch(rowd[m], 2 * sbf + 1, b, nx[m][1]);
  }
}

// One superblock sb of a wave's 16 rows (blocks cur, for each of NM matrices)
// against the activation image at ap (this lane's token row, 16 * (lane >> 4) in;
// arow: the lane's token is staged), added to acc with the superblock's scales.
template <int NM>
__device__ __forceinline__ void fp4_sb(const Fp4Blk (&cur)[NM][2], int sb, const uint8_t* ap, int64_t k, bool arow,
                                       const float* dx, v4f (&acc)[NM]) {
  const int b = (threadIdx.x & 63) >> 4;
  const v4f zf = {0.f, 0.f, 0.f, 0.f};
  v4f dd[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) dd[m] = zf;
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    int e8[NM];
    v8i bw[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) bw[m] = fp4_operand(cur[m][st], b, e8[m]);
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      u32x4 a0 = {0u, 0u, 0u, 0u}, a1 = {0u, 0u, 0u, 0u};
      if (arow) {
        const uint8_t* q = ap + pp * k + 256 * sb + 128 * st;
        a0 = *(const u32x4*)q;
        a1 = *(const u32x4*)(q + 64);
      }
      const v8i av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
#pragma unroll
      for (int m = 0; m < NM; ++m)
        dd[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bw[m], dd[m], 0, 4, 0, pp ? 131 : 127, 0,
                                                                  e8[m]);
    }
  }
  const v4f dxv = *(const v4f*)(dx + sb * 16 + 4 * b);
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[m][r] = fmaf(dxv[r], dd[m][r], acc[m][r]);
}

// The dot products of one wave: 16 rows (rowd[m] for each of NM matrices) over the
// superblocks [sb0, sb1), walked upwards (dir = 1) or downwards (dir = -1), against
// the activation image `act` (t_in tokens, those of tmask staged).  nx: the first
// superblock's blocks.  Result acc[m][r]: row (lane & 15) x token 4*(lane >> 4) + r.
template <int NM>
__device__ __forceinline__ void fp4_rows(const uint32_t* const (&rowd)[NM], int sb0, int sb1, int dir,
                                         Fp4Blk (&nx)[NM][2], const uint8_t* act, int64_t k, int t_in, uint32_t tmask,
                                         const float* dx, v4f (&acc)[NM]) {
  const int lane = threadIdx.x & 63, b = lane >> 4, tok = lane & 15;
  const bool arow = tok < t_in && ((tmask >> tok) & 1);
  const uint8_t* ap = act + (int64_t)tok * 2 * k + 16 * b;
  const v4f zf = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < NM; ++m) acc[m] = zf;
  const int n = sb1 - sb0;
  for (int it = 0; it < n; ++it) {
    const int sb = dir > 0 ? sb0 + it : sb1 - 1 - it;
    Fp4Blk cur[NM][2];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      cur[m][0] = nx[m][0];
      cur[m][1] = nx[m][1];
    }
    if (it + 1 < n) {
      const int sn = sb + dir;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        fp4_fetch(rowd[m], 2 * sn, b, nx[m][0]);
        fp4_fetch(rowd[m], 2 * sn + 1, b, nx[m][1]);
      }
    }
    fp4_sb<NM>(cur, sb, ap, k, arow, dx, acc);
  }
}

// The K walk through a per-wave LDS ring (rows a whole number of 16-byte chunks:
// K a multiple of 512).  A stage holds one superblock of the wave's 16 rows of
// each of NM matrices: per row the 9 chunks from the 16-byte boundary at or below
// the superblock's start (136 bytes at an offset of 0 or 8), 144 chunks per
// matrix, moved by global_load_lds (16 bytes per lane, CPS loads per wave and
// stage; lanes past the end re-read the last chunk).  Chunk cc of row r of matrix
// m sits in slot 144m + 9r + cc, so the 16 rows a read touches fall in distinct
// bank groups (9 is odd).  Lane (r, b) reads its 17-byte block of k-step st as the
// two slots from 4st + b (the block starts at dword 2P + st of them, P = the
// superblock's parity), i.e. the same five dwords the direct fetch takes.
// The ring's loads keep the default cache policy (lds_dma16_cached): two
// neighbouring superblock windows of a row share a 16-byte chunk (the 9-chunk
// windows overlap), and with the streaming (nt) hint that line was fetched again
// for the second window (the launch fetched 1.36x its weight bytes; cached, 1.02x:
// 1 token 35.6 -> 33.5 us, 2 tokens 63.6-64.1 -> 56.3-56.7 us, 4 tokens
// 122.8-124.1 -> 105.5-106 us).
template <int NM>
struct Fp4Ring {
  static constexpr int CPS = (NM * 144 + 63) / 64;   // DMA loads per wave and stage
  static constexpr int STAGE = CPS * 1024;           // LDS bytes of one stage
  const uint8_t* p[CPS];                             // this lane's chunk of each load, at row offset 0
  uint8_t* ring;
  int sb0, sb1, dir, n, issued, spare;
  __device__ __forceinline__ void init(const uint8_t* const (&grp)[NM], int64_t row_bytes, uint8_t* ring_, int sb0_,
                                       int sb1_, int dir_, int nsb) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int c = 0; c < CPS; ++c) {
      const int q = min(64 * c + lane, NM * 144 - 1), m = q / 144, rr = (q - 144 * m) / 9, cc = q - 144 * m - 9 * rr;
      p[c] = grp[m] + rr * row_bytes + 16 * cc;
    }
    ring = ring_;
    sb0 = sb0_;
    sb1 = sb1_;
    dir = dir_;
    n = sb1 - sb0;
    issued = 0;
    spare = sb0 < nsb ? sb0 : nsb - 1;
  }
  __device__ __forceinline__ int sb_of(int it) const { return dir > 0 ? sb0 + it : sb1 - 1 - it; }
  // the next superblock of the walk into its stage (past the walk: a valid one, unused,
  // so that the first RS stages can be issued unconditionally)
  template <int RS>
  __device__ __forceinline__ void issue() {
    const int64_t win = (int64_t)(136 * (issued < n ? sb_of(issued) : spare)) & ~(int64_t)15;
    uint8_t* dst = ring + (issued % RS) * STAGE;
#pragma unroll
    for (int c = 0; c < CPS; ++c) lds_dma16_cached(p[c] + win, dst + 1024 * c);
    ++issued;
  }
};

template <int NM, int RS>
__device__ __forceinline__ void fp4_rows_ring(Fp4Ring<NM>& rg, const uint8_t* act, int64_t k, int t_in,
                                              uint32_t tmask, const float* dx, v4f (&acc)[NM]) {
  constexpr int CPS = Fp4Ring<NM>::CPS;
  const int lane = threadIdx.x & 63, b = lane >> 4, tok = lane & 15, r = lane & 15;
  const bool arow = tok < t_in && ((tmask >> tok) & 1);
  const uint8_t* ap = act + (int64_t)tok * 2 * k + 16 * b;
  const v4f zf = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < NM; ++m) acc[m] = zf;
  for (int it = 0; it < rg.n; ++it) {
    wait_tiles<CPS, RS>(rg.issued - 1 - it);
    const uint8_t* stg = rg.ring + (it % RS) * Fp4Ring<NM>::STAGE;
    const int sb = rg.sb_of(it);
    const bool odd = sb & 1;
    Fp4Blk cur[NM][2];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4* s = (const u32x4*)(stg + 16 * (144 * m + 9 * r + 4 * st + b));
        const u32x4 u0 = s[0], u1 = s[1];
        uint32_t* d = cur[m][st].d;   // dwords st .. st + 4 of the pair (odd: 2 further), named one by one
        if (st == 0) {
          d[0] = odd ? u0.z : u0.x;
          d[1] = odd ? u0.w : u0.y;
          d[2] = odd ? u1.x : u0.z;
          d[3] = odd ? u1.y : u0.w;
          d[4] = odd ? u1.z : u1.x;
        } else {
          d[0] = odd ? u0.w : u0.y;
          d[1] = odd ? u1.x : u0.z;
          d[2] = odd ? u1.y : u0.w;
          d[3] = odd ? u1.z : u1.x;
          d[4] = odd ? u1.w : u1.y;
        }
      }
    fp4_sb<NM>(cur, sb, ap, k, arow, dx, acc);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0): the stage is read
    if (rg.issued < rg.n) rg.template issue<RS>();
  }
}

// Sum the KQ K-parts of each row group (fixed order) through LDS `red`
// ([row group][K part][64 lanes][NM * 4] fp32, wave = KQ * row group + part);
// returns true in the waves of part 0, whose acc then holds the totals.
template <int NM, int KQ>
__device__ __forceinline__ bool fp4_reduce(v4f (&acc)[NM], float* red) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  float* mine = red + ((size_t)wave * 64 + lane) * (NM * 4);
#pragma unroll
  for (int m = 0; m < NM; ++m) *(v4f*)(mine + 4 * m) = acc[m];
  __syncthreads();
  if (wave % KQ != 0) return false;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    v4f s = *(const v4f*)(mine + 4 * m);
#pragma unroll
    for (int q = 1; q < KQ; ++q) {
      const v4f o = *(const v4f*)(mine + (size_t)q * 64 * (NM * 4) + 4 * m);
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] += o[r];
    }
    acc[m] = s;
  }
  return true;
}

// gate/up + SwiGLU for 16 * 8 / KQ rows of the expert of slot blockIdx.y (KQ K parts
// per 16-row group; odd parts walk their superblocks downwards, so that a cache line
// shared by two neighbouring parts is read by both at about the same time)
template <int KQ, int RS>
__global__ void __launch_bounds__(MF_THREADS)
moe_fp4_gate_up_kernel(const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu, int64_t n_expert,
                       int64_t inter, int64_t hidden, const float* __restrict__ x, int t_real,
                       const int32_t* __restrict__ ids, int topk, float* __restrict__ h, float* __restrict__ gtap,
                       float* __restrict__ utap, const float* __restrict__ logits, int32_t* __restrict__ ids_out,
                       float* __restrict__ w_out) {
  extern __shared__ u32x4 smem4[];
  uint8_t* act = (uint8_t*)smem4;                           // [t_real][2 * hidden]
  float* dx = (float*)(act + (size_t)t_real * 2 * hidden);  // [hidden / 256][16]
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  // routed here: the logits first (loads complete in order: the selection then
  // waits for nothing after them)
  float raw[4];
  if (logits && wave < t_real) route_load<4>(logits + (int64_t)wave * n_expert, (int)n_expert, lane, raw);
  // the x of this thread's first two quantization items (they need no expert id):
  // requested before the ids and the weights, so that the quantization waits for
  // neither
  const int per_row = (int)(hidden / 16), total = t_real * per_row;
  float xv[2][16];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (j == 1 && total <= MF_THREADS) break;   // (uniform; the wait before the quantization is explicit)
    const int idx = min(tid + j * MF_THREADS, total - 1);
    const int r = idx / per_row, c = idx - r * per_row;
    const float4* p = (const float4*)(x + (int64_t)r * hidden) + 4 * c;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = p[q];
      xv[j][4 * q] = f.x;
      xv[j][4 * q + 1] = f.y;
      xv[j][4 * q + 2] = f.z;
      xv[j][4 * q + 3] = f.w;
    }
  }
  // x -> Q8_K codes -> FP8 halves in LDS (16 elements per thread, 16 lanes per block)
  const int nsb = (int)(hidden / 256);
  // Only the tokens of tm (the expert's), compacted in token order: row j of the
  // image and of the MFMA's A operand is the j-th token of tm.
  auto quantize = [&](uint32_t tm) {
    for (int idx0 = 0; idx0 < total; idx0 += MF_THREADS) {
      const int idx = idx0 + tid;
      const int r = idx / per_row, c = idx - r * per_row;
      if (idx < total && ((tm >> r) & 1)) {   // the same for all 16 lanes of a block
        const int jr = __popc(tm & ((1u << r) - 1));
        float v[16];
        if (idx0 < 2 * MF_THREADS) {
#pragma unroll
          for (int q = 0; q < 16; ++q) v[q] = idx0 == 0 ? xv[0][q] : xv[1][q];
        } else {
          const float4* p = (const float4*)(x + (int64_t)r * hidden) + 4 * c;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 f = p[q];
            v[4 * q] = f.x;
            v[4 * q + 1] = f.y;
            v[4 * q + 2] = f.z;
            v[4 * q + 3] = f.w;
          }
        }
        uint32_t w[4];
        int s;
        float d;
        q8_k_codes(v, w, s, d);
        stage_codes(w, act + (int64_t)jr * 2 * hidden, hidden, c >> 4, c & 15);
        if ((c & 15) == 0) dx[(c >> 4) * 16 + jr] = d;
      }
    }
  };
  for (int i = tid; i < nsb * 16; i += MF_THREADS) dx[i] = 0.0f;
  lds_barrier();
  int e;
  uint32_t mask;
  uint64_t smask;
  if (logits) {
    // routed here (n_expert <= 256): wave i takes token i of the chunk, with the
    // router's own selection and weights, into LDS; workgroup (0, 0) hands the
    // routing on to the later stages and the caller
    __shared__ int32_t s_rid[MF_MAXT * 8];
    __shared__ float s_rw[MF_MAXT * 8];
    if (wave < t_real) route_select<4>(raw, (int)n_expert, topk, lane, s_rid + wave * topk, s_rw + wave * topk);
    __syncthreads();
    const int npairs = t_real * topk;
    if (blockIdx.x == 0 && blockIdx.y == 0 && tid < npairs) {
      ids_out[tid] = s_rid[tid];
      w_out[tid] = s_rw[tid];
    }
    const int ep = lane < npairs ? s_rid[lane] : -1;
    if (!expert_tokens_of(ep, blockIdx.y, t_real, topk, e, mask, smask)) return;
  } else {
    if (!expert_tokens(ids, blockIdx.y, t_real, topk, n_expert, e, mask, smask)) return;
  }

  constexpr int RG = MF_WAVES / KQ;
  const int rg = wave / KQ, kq = wave % KQ, dir = (kq & 1) ? -1 : 1;
  const int64_t row = (int64_t)blockIdx.x * (16 * RG) + rg * 16 + (lane & 15);
  const int64_t row_bytes = hidden / 32 * 17;
  const uint32_t* const rowd[2] = {(const uint32_t*)(wg + ((int64_t)e * inter + row) * row_bytes),
                                   (const uint32_t*)(wu + ((int64_t)e * inter + row) * row_bytes)};
  const int sb0 = kq * nsb / KQ, sb1 = (kq + 1) * nsb / KQ;
  Fp4Blk nx[2][2];
  Fp4Ring<2> ring;
  if constexpr (RS > 0) {   // the wave's ring follows the activation image and scales
    const int64_t row0 = (int64_t)blockIdx.x * (16 * RG) + rg * 16;
    const uint8_t* const grp[2] = {wg + ((int64_t)e * inter + row0) * row_bytes, wu + ((int64_t)e * inter + row0) * row_bytes};
    const size_t roff = ((size_t)t_real * 2 * hidden + (size_t)nsb * 64 + 15) & ~(size_t)15;
    ring.init(grp, row_bytes, (uint8_t*)smem4 + roff + (size_t)wave * RS * Fp4Ring<2>::STAGE, sb0, sb1, dir, nsb);
#pragma unroll
    for (int j = 0; j < RS; ++j) ring.template issue<RS>();   // a fixed count: the compiler's waits stay exact
  } else {
    fp4_first<2>(rowd, dir > 0 ? sb0 : sb1 - 1, nsb, nx);
  }
  // quantize while the first superblocks stream in (quantizing before the weight
  // requests, during the routing, measured slower at 1-2 tokens)
  if constexpr (RS > 0) wait_vm<RS * Fp4Ring<2>::CPS>();   // x is in (loads complete in order)
  quantize(mask);
  const int ntok = __popc(mask);
  lds_barrier();   // the image is complete (a barrier with a full fence would wait for the weight loads)

  v4f acc[2];
  if constexpr (RS > 0) fp4_rows_ring<2, RS>(ring, act, hidden, ntok, 0xFFu, dx, acc);
  else fp4_rows<2>(rowd, sb0, sb1, dir, nx, act, hidden, ntok, 0xFFu, dx, acc);
  __syncthreads();   // the activation image is dead: the reduction reuses its LDS
  if (!fp4_reduce<2, KQ>(acc, (float*)smem4)) return;

  const int b = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int j = 4 * b + r;   // compacted row -> the token
    if (j < ntok) {
      const int i = nth_bit(mask, j);
      const float g = acc[0][r], u = acc[1][r], hv = g / (1.0f + expf(-g)) * u;
      for (int k = 0; k < topk; ++k) {
        if ((smask >> (8 * i + k)) & 1) {
          const int64_t o = (int64_t)(i * topk + k) * inter + row;
          h[o] = hv;
          if (gtap) gtap[o] = g;
          if (utap) utap[o] = u;
        }
      }
    }
  }
}

// down projection for 16 * 8 / KQ rows of the expert of slot blockIdx.y: d[pair][r] for
// every slot naming it.  hhat of the expert's tokens is quantized here from the
// first slot's h row (or taken from in_hq); the workgroup of row block 0 writes
// the Q8_K blocks to hq_tap for every slot naming the expert.
template <int KQ, int RS>
__global__ void __launch_bounds__(MF_THREADS)
moe_fp4_down_kernel(const uint8_t* __restrict__ wd, int64_t n_expert, int64_t hidden, int64_t inter,
                    const float* __restrict__ h, const uint8_t* __restrict__ in_hq, uint8_t* __restrict__ hq_tap,
                    int t_real, const int32_t* __restrict__ ids, int topk, float* __restrict__ dpair) {
  extern __shared__ u32x4 smem4[];
  uint8_t* act = (uint8_t*)smem4;                          // [t_real][2 * inter]
  float* dx = (float*)(act + (size_t)t_real * 2 * inter);  // [inter / 256][16]
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  int e;
  uint32_t mask;
  uint64_t smask;
  if (!expert_tokens(ids, blockIdx.y, t_real, topk, n_expert, e, mask, smask)) return;

  constexpr int RG = MF_WAVES / KQ;
  const int nsb = (int)(inter / 256), rg = wave / KQ, kq = wave % KQ, dir = (kq & 1) ? -1 : 1;
  const int64_t row = (int64_t)blockIdx.x * (16 * RG) + rg * 16 + (lane & 15);
  const int64_t row_bytes = inter / 32 * 17;
  const uint32_t* const rowd[1] = {(const uint32_t*)(wd + ((int64_t)e * hidden + row) * row_bytes)};
  const int sb0 = kq * nsb / KQ, sb1 = (kq + 1) * nsb / KQ;
  Fp4Blk nx[1][2];
  Fp4Ring<1> ring;
  if constexpr (RS > 0) {   // the wave's ring follows the activation images and scales
    const int64_t row0 = (int64_t)blockIdx.x * (16 * RG) + rg * 16;
    const uint8_t* const grp[1] = {wd + ((int64_t)e * hidden + row0) * row_bytes};
    const size_t roff = ((size_t)t_real * 2 * inter + (size_t)nsb * 64 + 15) & ~(size_t)15;
    ring.init(grp, row_bytes, (uint8_t*)smem4 + roff + (size_t)wave * RS * Fp4Ring<1>::STAGE, sb0, sb1, dir, nsb);
#pragma unroll
    for (int j = 0; j < RS; ++j) ring.template issue<RS>();
  } else {
    fp4_first<1>(rowd, dir > 0 ? sb0 : sb1 - 1, nsb, nx);
  }
  const int hrb = nsb * 292;
  auto first_pair = [&](int i) { return i * topk + __ffs((unsigned)(smask >> (8 * i)) & 0xFFu) - 1; };
  const bool tap = hq_tap && blockIdx.x == 0;

  for (int i = tid; i < nsb * 16; i += MF_THREADS) dx[i] = 0.0f;
  __syncthreads();
  const int ntok = __popc(mask), per_row = (int)(inter / 16), total = ntok * per_row;
  for (int idx0 = 0; idx0 < total; idx0 += MF_THREADS) {
    const int idx = idx0 + tid;
    if (idx < total) {
      const int j = idx / per_row, c = idx - j * per_row, i = nth_bit(mask, j), sb = c >> 4, l16 = c & 15;
      const int64_t src = first_pair(i);
      uint32_t w[4];
      int s;
      float d;
      if (in_hq) {
        const uint8_t* blk = in_hq + src * hrb + (int64_t)sb * 292;   // 4-byte aligned
        const uint32_t* q = (const uint32_t*)(blk + 4 + 16 * l16);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) w[jj] = q[jj];
        d = *(const float*)blk;
        s = *(const int16_t*)(blk + 260 + 2 * l16);
      } else {
        const float4* p = (const float4*)(h + src * inter) + 4 * c;
        float v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 f = p[q];
          v[4 * q] = f.x;
          v[4 * q + 1] = f.y;
          v[4 * q + 2] = f.z;
          v[4 * q + 3] = f.w;
        }
        q8_k_codes(v, w, s, d);
      }
      stage_codes(w, act + (int64_t)i * 2 * inter, inter, sb, l16);
      if (l16 == 0) dx[sb * 16 + i] = d;
      if (tap) {
        for (int k = 0; k < topk; ++k)
          if ((smask >> (8 * i + k)) & 1) q8_k_store(w, s, d, l16, hq_tap + (int64_t)(i * topk + k) * hrb + sb * 292);
      }
    }
  }
  __syncthreads();

  v4f acc[1];
  if constexpr (RS > 0) fp4_rows_ring<1, RS>(ring, act, inter, t_real, mask, dx, acc);
  else fp4_rows<1>(rowd, sb0, sb1, dir, nx, act, inter, t_real, mask, dx, acc);
  __syncthreads();
  if (!fp4_reduce<1, KQ>(acc, (float*)smem4)) return;

  const int b = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 4 * b + r;
    if (i < t_real && ((mask >> i) & 1)) {
      for (int k = 0; k < topk; ++k)
        if ((smask >> (8 * i + k)) & 1) dpair[(int64_t)(i * topk + k) * hidden + row] = acc[0][r];
    }
  }
}

// Down and the weighted combine in one launch.  Workgroup (x, i) owns 16 * R output
// rows of token i for every slot of that token: wave 2s + p takes slot s's expert
// over K part p (of 2, odd parts walking downwards as above) for its R row groups,
// so the slots' down values of a row meet in LDS and are summed in slot order there
// (ft_moe_combine's arithmetic), and no per-pair rows go out.  The prologue
// quantizes the token's h rows, one per slot, to Q8_K (or takes in_hq) into
// FP8-half images.  A slot repeating an earlier slot's expert, in this token or
// another, is computed again (same d, its own weight): the tokens' workgroups are
// independent.
constexpr int MF_DC_WAVES = 16;   // 8 slots x 2 K parts
// byte offset of the down + combine launch's s_d: past the images and scales and
// past fp4_reduce's K-part sums
__host__ __device__ inline size_t fp4_dc_sd_off(int64_t inter, int r) {
  const size_t img = (size_t)8 * 2 * inter + (size_t)8 * (inter / 256) * 16 * 4;
  const size_t red = (size_t)MF_DC_WAVES * 64 * r * 4 * 4;
  return img > red ? img : red;
}
// NW > 0: every superblock of a wave's K part (at most NW) is requested right after
// the quantization, all at once, and each superblock's dot waits only for its own
// loads (loads complete in order; every wave issues the same loads).  Requested
// before the quantization, the loads of the whole layer's down matrices held up
// the quantization behind their issue; one superblock of lookahead (NW = 0, longer
// K parts) pays a full memory latency per superblock.
template <int NW, int R>
__global__ void __launch_bounds__(64 * MF_DC_WAVES)
moe_fp4_down_combine_kernel(const uint8_t* __restrict__ wd, int64_t n_expert, int64_t hidden, int64_t inter,
                            const float* __restrict__ h, const uint8_t* __restrict__ in_hq,
                            uint8_t* __restrict__ hq_tap, const int32_t* __restrict__ ids,
                            const float* __restrict__ ew, int topk, float* __restrict__ d_tap,
                            float* __restrict__ y) {
  extern __shared__ u32x4 smem4[];
  const int nsb = (int)(inter / 256);
  uint8_t* act = (uint8_t*)smem4;                               // [8][2 * inter]
  float* dx = (float*)(act + (size_t)8 * 2 * inter);            // [8][nsb][16]
  // s_d [8][16 * R] past both the images and the K-part sums (fp4_reduce's area from
  // offset 0): a part-0 wave writes it while others still read their partners' sums
  float* s_d = (float*)smem4 + fp4_dc_sd_off(inter, R) / 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int s = wave >> 1, kq = wave & 1, dir = kq ? -1 : 1;
  const int hrb = nsb * 292;
  const int64_t p0 = (int64_t)blockIdx.y * topk;                // the token's first pair
  const bool live = s < topk;
  // NW > 0: slots past topk read slot 0's rows (unused), so that every wave issues the same loads
  const int e = live ? clamp_id(ids[p0 + s], n_expert) : (NW > 0 ? clamp_id(ids[p0], n_expert) : 0);
  const int64_t row = (int64_t)blockIdx.x * (16 * R) + (lane & 15);   // + 16 r for row group r
  const int64_t row_bytes = inter / 32 * 17;
  const int sb0 = kq * nsb / 2, sb1 = (kq + 1) * nsb / 2, n = sb1 - sb0;
  const uint32_t* rowd[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rowd[r] = (const uint32_t*)(wd + ((int64_t)e * hidden + row + 16 * r) * row_bytes);
  Fp4Blk nx[R][2];
  if (NW == 0 && live) fp4_first<R>(rowd, dir > 0 ? sb0 : sb1 - 1, nsb, nx);   // slots past topk stream nothing

  // every slot's h row -> Q8_K codes -> FP8 halves (16 elements per thread)
  for (int i = tid; i < 8 * nsb * 16; i += 64 * MF_DC_WAVES) dx[i] = 0.0f;
  __syncthreads();
  const int per_row = (int)(inter / 16), total = topk * per_row;
  for (int idx = tid; idx < total; idx += 64 * MF_DC_WAVES) {   // a block's 16 lanes stay together
    const int j = idx / per_row, c = idx - j * per_row, sb = c >> 4, l16 = c & 15;
    uint32_t w[4];
    int sm;
    float d;
    if (in_hq) {
      const uint8_t* blk = in_hq + (p0 + j) * hrb + (int64_t)sb * 292;
      const uint32_t* q = (const uint32_t*)(blk + 4 + 16 * l16);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) w[jj] = q[jj];
      d = *(const float*)blk;
      sm = *(const int16_t*)(blk + 260 + 2 * l16);
    } else {
      const float4* p = (const float4*)(h + (p0 + j) * inter) + 4 * c;
      float v[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 f = p[q];
        v[4 * q] = f.x;
        v[4 * q + 1] = f.y;
        v[4 * q + 2] = f.z;
        v[4 * q + 3] = f.w;
      }
      q8_k_codes(v, w, sm, d);
    }
    stage_codes(w, act + (int64_t)j * 2 * inter, inter, sb, l16);
    if (l16 == 0) dx[(j * nsb + sb) * 16] = d;
    if (hq_tap && blockIdx.x == 0) q8_k_store(w, sm, d, l16, hq_tap + (p0 + j) * hrb + sb * 292);
  }
  Fp4Blk wb[NW > 0 ? NW : 1][R][2];
  if constexpr (NW > 0) {
#pragma unroll
    for (int j = 0; j < NW; ++j) {   // superblock j in walk order (past the part: a valid one, unused)
      int sb = dir > 0 ? sb0 + j : sb1 - 1 - j;
      sb = sb < 0 ? 0 : (sb < nsb ? sb : nsb - 1);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        fp4_fetch(rowd[r], 2 * sb, lane >> 4, wb[j][r][0]);
        fp4_fetch(rowd[r], 2 * sb + 1, lane >> 4, wb[j][r][1]);
      }
    }
    lds_barrier();   // (a barrier with a full fence would wait for those loads)
  } else {
    __syncthreads();
  }

  v4f acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (NW > 0) {
    const int tok = lane & 15;
    const uint8_t* ap = act + (size_t)s * 2 * inter + (int64_t)tok * 2 * inter + 16 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      if (live && j < n)
        fp4_sb<R>(wb[j], dir > 0 ? sb0 + j : sb1 - 1 - j, ap, inter, tok == 0, dx + (size_t)s * nsb * 16, acc);
    }
  } else {
    if (live) fp4_rows<R>(rowd, sb0, sb1, dir, nx, act + (size_t)s * 2 * inter, inter, 1, 1u, dx + (size_t)s * nsb * 16, acc);
  }
  __syncthreads();   // the images are dead: the K-part sums reuse their LDS
  if (fp4_reduce<R, 2>(acc, (float*)smem4)) {
    // part-0 wave of slot s: lanes 0..15 hold row (lane & 15) of each row group
    if (live && lane < 16) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        s_d[s * 16 * R + 16 * r + lane] = acc[r][0];
        if (d_tap) d_tap[(p0 + s) * hidden + row + 16 * r] = acc[r][0];
      }
    }
  }
  __syncthreads();
  if (tid < 16 * R) {
    float sum = 0.0f;
    for (int k = 0; k < topk; ++k) sum = fmaf(ew[p0 + k], s_d[k * 16 * R + tid], sum);
    y[(int64_t)blockIdx.y * hidden + (int64_t)blockIdx.x * 16 * R + tid] = sum;
  }
}

// LDS bytes of one launch: the activation image and scales, or the K-quarter
// partials, whichever is larger
static size_t fp4_lds(int t, int64_t k, int nm) {
  const size_t img = (size_t)t * 2 * k + (size_t)(k / 256) * 16 * 4;
  const size_t red = (size_t)MF_WAVES * 64 * nm * 4 * 4;
  return img > red ? img : red;
}

}  // namespace ftk

using namespace ftk;

// Direct-route stages for MXFP4 x Q8_K.  Shapes: hidden and inter multiples of
// 256 (so every workgroup's rows exist); tokens in chunks of up to 8 that fit
// 64 KiB of LDS.  down: 2 K parts x 4 row groups.
constexpr int MF_KQ_DN = 2;
static int fp4_chunk(int64_t k, int nm) {
  int cs = MF_MAXT;
  while (cs > 1 && fp4_lds(cs, k, nm) > 65536) cs /= 2;
  return fp4_lds(cs, k, nm) > 65536 ? 0 : cs;
}

template <int KQ, int RS>
static hipError_t fp4_gate_up_kq(const MoeArgs& a, int c0, int tc, hipStream_t st) {
  const dim3 grid((unsigned)(a.inter / (16 * MF_WAVES / KQ)), (unsigned)(tc * a.topk));
  const size_t p0 = (size_t)c0 * a.topk;
  size_t lds = fp4_lds(tc, a.hidden, 2);
  if (RS > 0) {
    const size_t ring = (((size_t)tc * 2 * a.hidden + (size_t)(a.hidden / 256) * 64 + 15) & ~(size_t)15) +
                        (size_t)MF_WAVES * RS * Fp4Ring<2>::STAGE;
    lds = ring > lds ? ring : lds;
    // (the kernel's static LDS, the routing, counts against the same 160 KiB)
    static const bool attr = hipFuncSetAttribute((const void*)moe_fp4_gate_up_kernel<KQ, RS>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, 159 * 1024) == hipSuccess;
    if (!attr || lds > 159 * 1024) return hipErrorInvalidConfiguration;
  }
  hipLaunchKernelGGL((moe_fp4_gate_up_kernel<KQ, RS>), grid, dim3(MF_THREADS), lds, st,
                     (const uint8_t*)a.w_gate, (const uint8_t*)a.w_up, a.n_expert, a.inter, a.hidden,
                     a.x + (size_t)c0 * a.hidden, tc, a.ids + p0, a.topk, a.h + p0 * a.inter,
                     a.g_tap ? a.g_tap + p0 * a.inter : nullptr, a.u_tap ? a.u_tap + p0 * a.inter : nullptr,
                     a.logits ? a.logits + (size_t)c0 * a.n_expert : nullptr,
                     a.logits ? const_cast<int32_t*>(a.ids) + p0 : nullptr,
                     a.logits ? const_cast<float*>(a.ew) + p0 : nullptr);
  return hipGetLastError();
}

// gate/up K parts: 2 (each row's K in two halves: one cache line shared per row)
// when that still gives a workgroup per CU, else 4 (more workgroups, three shared
// lines per row).  At 1 token of the 256 x 2048 x 4096 layer (one workgroup per CU)
// 2 parts measure 38.0-38.3 against 38.4-38.8 us per layer; at 2-8 tokens 2 parts
// win by 5-10%.  With K a multiple of 512 the K walk runs on the LDS ring: 2 stages
// per wave at 1 token (layer 38.2-38.4 -> 37.0-37.2 us), 1 stage from 2 tokens,
// where the smaller ring keeps two workgroups per CU (2 / 4 / 8 tokens 69.4 / 130
// / 235 -> 68.1-69.0 / 127.7-128.2 / 230-233 us; 2 stages there: no gain, 3 stages
// at 1 token: no gain).  The same ring in the per-expert down launch was slower
// (2-8 tokens +2-5%).
hipError_t ftk_launch_moe_fp4_gate_up(const MoeArgs& a, hipStream_t st) {
  const int cs = fp4_chunk(a.hidden, 2);
  if (cs < 1 || a.hidden % 256 || a.inter % 256) return hipErrorInvalidValue;
  for (int64_t c0 = 0; c0 < a.t; c0 += cs) {
    const int tc = (int)(a.t - c0 < cs ? a.t - c0 : cs);
    const int64_t wgs2 = a.inter / (16 * MF_WAVES / 2) * tc * a.topk;
    const bool k2 = wgs2 >= (int64_t)ftk_num_cus();
    hipError_t err;
    if (a.hidden % 512) err = k2 ? fp4_gate_up_kq<2, 0>(a, (int)c0, tc, st) : fp4_gate_up_kq<4, 0>(a, (int)c0, tc, st);
    else if (tc == 1) err = k2 ? fp4_gate_up_kq<2, 2>(a, (int)c0, tc, st) : fp4_gate_up_kq<4, 2>(a, (int)c0, tc, st);
    else err = k2 ? fp4_gate_up_kq<2, 1>(a, (int)c0, tc, st) : fp4_gate_up_kq<4, 1>(a, (int)c0, tc, st);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// down + combine in one launch at 1-2 tokens (top-k <= 8): workgroup (x, i) takes
// 16 * R rows of token i, R = 1 at one token (a workgroup per CU), 2 at two (the
// quantization of a token's h rows shared by twice the rows; 256 workgroups
// again).  Against the per-expert down launch and the combine launch: 2 tokens
// 68.1-68.6 -> 64.0-64.3 us per layer; 3, 5 and 8 tokens (1.5, 2.5 and 4 rounds
// of workgroups) were 3-8 us slower and 4 tokens even, so from 3 tokens the layer
// keeps the two launches.
constexpr int MF_DC_MAXT = 2;
static size_t fp4_dc_lds(int64_t inter, int r) { return fp4_dc_sd_off(inter, r) + (size_t)8 * 16 * r * 4; }
bool ftk_moe_fp4_down_combine_ok(const MoeArgs& a) {
  const int r = a.t == 1 ? 1 : 2;
  return a.t >= 1 && a.t <= MF_DC_MAXT && a.topk <= 8 && a.hidden % (16 * r) == 0 && a.inter % 256 == 0 &&
         fp4_dc_lds(a.inter, r) <= 65536;
}
template <int R>
static hipError_t fp4_down_combine_r(const MoeArgs& a, hipStream_t st) {
  const int nw = (int)(a.inter / 256 + 1) / 2;   // superblocks of a wave's K part, at most
  auto kern = nw == 0 ? moe_fp4_down_combine_kernel<0, R> : nw <= 1 ? moe_fp4_down_combine_kernel<1, R>
            : nw <= 2 ? moe_fp4_down_combine_kernel<2, R> : nw <= 4 ? moe_fp4_down_combine_kernel<4, R>
            : moe_fp4_down_combine_kernel<0, R>;
  hipLaunchKernelGGL(kern, dim3((unsigned)(a.hidden / (16 * R)), (unsigned)a.t), dim3(64 * MF_DC_WAVES),
                     fp4_dc_lds(a.inter, R), st, (const uint8_t*)a.w_down, a.n_expert, a.hidden, a.inter, a.h,
                     (const uint8_t*)a.in_hq, (uint8_t*)a.hq_tap, a.ids, a.ew, a.topk, a.d_tap, a.y);
  return hipGetLastError();
}
hipError_t ftk_launch_moe_fp4_down_combine(const MoeArgs& a, hipStream_t st) {
  if (!ftk_moe_fp4_down_combine_ok(a)) return hipErrorInvalidValue;
  return a.t == 1 ? fp4_down_combine_r<1>(a, st) : fp4_down_combine_r<2>(a, st);
}

hipError_t ftk_launch_moe_fp4_down(const MoeArgs& a, hipStream_t st) {
  const int cs = fp4_chunk(a.inter, 1);
  if (cs < 1 || a.hidden % 256 || a.inter % 256) return hipErrorInvalidValue;
  const int64_t hrb = a.inter / 256 * 292;
  for (int64_t c0 = 0; c0 < a.t; c0 += cs) {
    const int tc = (int)(a.t - c0 < cs ? a.t - c0 : cs);
    const dim3 grid((unsigned)(a.hidden / (16 * MF_WAVES / MF_KQ_DN)), (unsigned)(tc * a.topk));
    const size_t p0 = (size_t)c0 * a.topk;
    // K walk on the LDS ring (one stage per wave, cached loads) up to 5 tokens:
    // 3 / 4 / 5 tokens 87.1-88.7 / 107.7-107.8 / 130.0-130.3 -> 86.1-86.4 /
    // 104.9-105.7 / 128.5-128.6 us per layer; at 8 tokens its LDS halves the
    // workgroups per CU (191 -> 197 us), and two stages were slower throughout
    size_t lds = fp4_lds(tc, a.inter, 1);
    const bool ring = a.inter % 512 == 0 && tc <= 5;
    if (ring) {
      const size_t r = (((size_t)tc * 2 * a.inter + (size_t)(a.inter / 256) * 64 + 15) & ~(size_t)15) +
                       (size_t)MF_WAVES * Fp4Ring<1>::STAGE;
      lds = r > lds ? r : lds;
      static const bool attr = hipFuncSetAttribute((const void*)moe_fp4_down_kernel<MF_KQ_DN, 1>,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, 159 * 1024) == hipSuccess;
      if (!attr || lds > 159 * 1024) return hipErrorInvalidConfiguration;
    }
    auto kern = ring ? moe_fp4_down_kernel<MF_KQ_DN, 1> : moe_fp4_down_kernel<MF_KQ_DN, 0>;
    hipLaunchKernelGGL(kern, grid, dim3(MF_THREADS), lds, st,
                       (const uint8_t*)a.w_down, a.n_expert, a.hidden, a.inter, a.h + p0 * a.inter,
                       a.in_hq ? (const uint8_t*)a.in_hq + p0 * hrb : nullptr,
                       a.hq_tap ? (uint8_t*)a.hq_tap + p0 * hrb : nullptr, tc, a.ids + p0, a.topk,
                       a.dpair + p0 * a.hidden);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}
