// Routed prefill linear (T > 64), MFMA kernel: per budget group b,
//   Y_b = X_b . W^(b)^T,   W^(b)[n, k] = sum_{j <= b} (z_jng + s_jng * q_jnk)
// with the summed slices dequantized to bfloat16 once per tile and multiplied on
// 32x32x16 bf16 MFMA with float32 accumulation.
//
// MoBiQuant explainer (gist.science, English), sections 2.A and 4: the summed slices are
// the token's weight and prefill cost grows with sequence length, so this path is a dense
// contraction.  The pages' kernel uses 1-bit binary tensor-core products on another
// vendor's GPU; CDNA4 has no 1-bit MFMA, so the slices are summed in float32 once per
// (tile, weight), rounded once to bfloat16 and fed to bf16 MFMA.
//
// Tiling.  A tile is BM tokens of one budget group (256, or 128 for a group's short
// remainder and for float32 activations) x 256 outputs, on 8 waves.  Wave w runs on SIMD
// w % 4; the two waves of a SIMD share column block wn = w & 3 (64 outputs) and split the
// tile's tokens (wm = w >> 2) and the block's dequantization (each dequantizes 32 of the
// 64 outputs).  Dequantized chunks are exchanged through LDS as ready-made MFMA B
// operands; activations are staged through LDS in chunks of 64 inputs (rows of 128 bytes,
// 16-byte pieces swizzled so operand reads are free of bank conflicts).
//
// Dequantization.  Each 2-bit field is turned into a float16 pair (o + q_e, o + q_e+1) by
// one AND-OR with an exponent pattern whose unit in the last place is the field's weight;
// the offsets are folded into a per-(row, group) constant C_o = sum_j z_j - o sum_j s_j,
// and each slice adds s_j * v_j with one mixed-precision FMA per weight (float16 inputs,
// float32 accumulate).  (A float16 dot2 would pair two slices per instruction, but DOT
// results need wait states before VALU reads that cost as much as it saves.)
//
// Pipeline per chunk: each group of MFMAs (one 32-row block, both column halves) is
// fenced around half of the dequantization of chunk q + 1, so one wave's VALU work runs
// in the shadow of the other wave's MFMAs; codes, params and activations of chunk q + 2
// load during chunk q, so the loop has no load it waits on at once.

#include "mbq_internal.h"

namespace mbq {
namespace {

constexpr int kBN = 256;   // outputs per tile

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Field f = 0..3 of each half-word's low byte: mask and float16 exponent pattern
// 2^(10 - 2f), whose unit in the last place is the field's weight 4^f.
constexpr uint32_t kMask[4] = {0x00030003u, 0x000C000Cu, 0x00300030u, 0x00C000C0u};
constexpr float kOff[4] = {1024.f, 256.f, 64.f, 16.f};

__device__ __forceinline__ float fmix(uint32_t v, int half, uint32_t sw, float c) {
  const half2_t vv = __builtin_bit_cast(half2_t, v);
  const half2_t ss = __builtin_bit_cast(half2_t, sw);
  return fmaf(float(half ? vv[1] : vv[0]), float(ss[0]), c);
}

__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  const bf16x2_t p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 32x32x16 bf16 MFMA: A lane l = row l % 32, k 8 (l / 32) .. + 7; B lane l = column
// l % 32, same k; D lane l = column l % 32, rows 8 (v / 4) + 4 (l / 32) + v % 4.  (The
// 32x32 forms accumulate in place, which keeps 256 accumulators in the AGPRs.)
__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

struct Magic {
  uint32_t m[4];  // float16 pairs 1024, 256, 64, 16 (vector registers)
};

// Per row block constants of one chunk: C_o = sum_j z_j - o sum_j s_j for the four field
// offsets, and the slices' param words (scale in the low half, used by the mixed FMAs).
template <int B>
struct Consts {
  float c[4];
  uint32_t p[B];
};

template <int B>
__device__ __forceinline__ Consts<B> consts(const uint32_t (&p)[B]) {
  float Z = 0.f, Ss = 0.f;
#pragma unroll
  for (int j = 0; j < B; ++j) {
    const half2_t h = __builtin_bit_cast(half2_t, p[j]);
    Ss += float(h[0]);
    Z += float(h[1]);
  }
  Consts<B> k;
#pragma unroll
  for (int i = 0; i < 4; ++i) k.c[i] = fmaf(-Ss, kOff[i], Z);
#pragma unroll
  for (int j = 0; j < B; ++j) k.p[j] = p[j];
  return k;
}

// The code words of one row block brought into position for half H of their 16 inputs:
// H = 0 keeps the low byte of each half-word (inputs e = 0..7 of the word), H = 1 shifts
// the high byte (e = 8..15) down.
template <int B>
struct Prep {
  uint32_t w[B];
};

template <int B, int H>
__device__ __forceinline__ Prep<B> prep(const uint32_t (&w)[B]) {
  Prep<B> p;
#pragma unroll
  for (int j = 0; j < B; ++j) p.w[j] = w[j] >> (8 * H);
  return p;
}

// bf16 pair f (k slots 2f, 2f + 1) of a prepared row block: W = C_o + sum_j s_j v_j, one
// mixed-precision FMA per slice and weight (float16 operands, float32 accumulate; each
// product is exact, so only the additions round).  Split in two halves so that each half
// fits in the shadow of one MFMA: the float16 fields and the even input, then the odd
// input and the bf16 rounding.  (The field extraction, (w & mask) | magic, is one
// v_and_or_b32 with the mask in a scalar and the magic in a vector register.)
template <int B>
struct Half {
  uint32_t v[B];
  float lo;
};

template <int B>
__device__ __forceinline__ Half<B> pair_a(const Prep<B>& p, const Consts<B>& k, const Magic& mg, int f) {
  Half<B> h;
  float lo = k.c[f];
#pragma unroll
  for (int j = 0; j < B; ++j) {
    h.v[j] = (p.w[j] & kMask[f]) | mg.m[f];
    lo = fmix(h.v[j], 0, k.p[j], lo);
  }
  h.lo = lo;
  return h;
}

template <int B>
__device__ __forceinline__ uint32_t pair_b(const Half<B>& h, const Consts<B>& k, int f) {
  float hi = k.c[f];
#pragma unroll
  for (int j = 0; j < B; ++j) hi = fmix(h.v[j], 1, k.p[j], hi);
  return pk_bf16(h.lo, hi);
}

template <int B>
__device__ __forceinline__ uint32_t pair(const Prep<B>& p, const Consts<B>& k, const Magic& mg, int f) {
  return pair_b<B>(pair_a<B>(p, k, mg, f), k, f);
}

struct TileArgs {
  const uint8_t* packed;
  uint32_t ss, po;        // slice stride, params offset (bytes)
  int N, KB, NG, NB, gshift, NQ, T;
  const void* x;
  uint32_t x_bytes, x_row;  // bytes of x, bytes per token row
  const int32_t* perm;
  void* y;
  int y_bf16;
  // low-rank side path (lr_r == 0: none): u [lr_ks x T x lr_r] float32 (chunks of K,
  // summed in order), B [N x lr_r] bf16
  const float* lr_u;
  const uint16_t* lr_b;
  int lr_r, lr_ks;
};

// Epilogue: a wave's outputs are staged in LDS as rows of 64 values (+16 bytes of
// padding against bank conflicts), PM MFMA row blocks per pass, then stored as 16-byte
// pieces of the output rows (8 bf16 or 4 float32 values of one token).  Lane holds rows
// 32 i + 8 (v / 4) + 4 c2 + v % 4 of the wave's tokens, column 32 k + col of its block.
// Rows of the output that are not 16-byte aligned, and the right edge, are stored per
// value.  Called after a barrier that ended all use of the LDS staging area.
template <int MB, int WM, bool YBF16>
__device__ __forceinline__ void store_tile(const f32x16_t (&acc)[MB][2], const TileArgs& a,
                                           const int32_t* tokT, uint8_t* lds, int wave, int wn,
                                           int wm, int lane, int n0) {
  constexpr int ES = YBF16 ? 2 : 4;
  constexpr int RB = 64 * ES + 16;                   // staged row bytes
  constexpr int PM = YBF16 ? 2 : 1;                  // row blocks per pass
  constexpr int PPR = 64 * ES / 16;                  // 16-byte pieces per row
  constexpr int PER = 16 / ES;                       // values per piece
  const int col = lane & 31, c2 = lane >> 5;
  const bool vec_ok = ((a.N * ES) & 15) == 0;
  uint8_t* stg = lds + wave * (PM * 32 * RB);
#pragma unroll
  for (int i0 = 0; i0 < MB; i0 += PM) {
#pragma unroll
    for (int d = 0; d < PM; ++d)
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rl = 32 * d + 8 * (v >> 2) + 4 * c2 + (v & 3);
          uint8_t* dst = stg + rl * RB + (32 * k + col) * ES;
          if constexpr (YBF16) *reinterpret_cast<uint16_t*>(dst) = uint16_t(pk_bf16(acc[i0 + d][k][v], 0.f));
          else *reinterpret_cast<float*>(dst) = acc[i0 + d][k][v];
        }
    // PM * 32 rows x PPR pieces = 512 pieces: 8 per lane
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int pp = lane + 64 * it;
      const int rl = pp / PPR, pc = pp % PPR;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + rl * RB + 16 * pc);
      const int t = tokT[WM * wm + 32 * i0 + rl];
      if (t < 0) continue;
      const int c0 = n0 + 64 * wn + pc * PER;
      uint8_t* yrow = static_cast<uint8_t*>(a.y) + size_t(t) * a.N * ES;
      if (vec_ok && c0 + PER <= a.N) {
        *reinterpret_cast<u32x4_t*>(yrow + size_t(c0) * ES) = v;
      } else {
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          if (c0 + e >= a.N) break;
          if constexpr (YBF16) reinterpret_cast<uint16_t*>(yrow)[c0 + e] = uint16_t(v[e >> 1] >> (16 * (e & 1)));
          else reinterpret_cast<uint32_t*>(yrow)[c0 + e] = v[e];
        }
      }
    }
  }
}

// LDS map (BM tokens per tile; ABUF = BM * 128 bytes per activation chunk):
//   [0, 2 ABUF)               activation chunks, two buffers of BM rows x 128 bytes
//   [2 ABUF, + 64 KiB)        dequantized weights, two buffers x 4 column blocks x 2
//                             halves x 4 steps x 1 KiB (one MFMA B operand each)
//   [2 ABUF + 64 KiB, + 1 KiB) row -> token table
// The epilogue reuses [0, 2 ABUF + 64 KiB) to stage the outputs.
template <bool XBF16>
constexpr int lds_bytes() {
  return 2 * (XBF16 ? 256 : 128) * 128 + 65536 + 1024;
}

template <int B, bool XBF16, int BM>
__device__ __forceinline__ void prefill_tile(const TileArgs& a, int start, int rows, int n0,
                                             uint8_t* lds) {
  constexpr int WM = BM / 2;              // tokens per wave
  constexpr int MB = WM / 32;             // 32-row MFMA blocks per wave
  constexpr int ABUF = BM * 128;
  constexpr int BX = 2 * ABUF, TOK = BX + 65536;
  const int tid = threadIdx.x;
  // wave w runs on SIMD w % 4: the two waves of a SIMD share column block wn and split
  // the tile's tokens (wm) and the block's dequantization (column half wm)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wn = wave & 3, wm = wave >> 2;
  const int col = lane & 31, c2 = lane >> 5, r = lane & 15, hi = (lane >> 4) & 1;

  // ---- row -> token table (out-of-contract perm entries are never stored)
  int32_t* tokT = reinterpret_cast<int32_t*>(lds + TOK);
  if (tid < BM) {
    const int t = tid < rows ? a.perm[start + tid] : -1;
    tokT[tid] = (t >= 0 && t < a.T) ? t : -1;
  }

  // ---- weights this wave dequantizes: column half wm (32 outputs = row blocks
  // 4 wn + 2 wm + {0, 1}) of column block wn.  Lane (c2, col) takes row r of block
  // 4 wn + 2 wm + hi and, of each chunk, the code words of lanes 16 (2 c2 + t) + r of the
  // packed tile, t = 0, 1.  Row blocks past the last are clamped (never stored).
  const int nb = min(n0 / 16 + 4 * wn + 2 * wm + hi, a.NB - 1);
  const uint32_t code_voff = uint32_t(nb) * uint32_t(a.KB) * kTileBytes + 512u * c2 + 16u * r;
  const uint32_t par_voff = a.po + uint32_t(nb) * uint32_t(a.NG) * 64u + 4u * r;
  __amdgpu_buffer_rsrc_t rs[B];
#pragma unroll
  for (int j = 0; j < B; ++j) rs[j] = rsrc(a.packed + uint64_t(j) * a.ss, a.ss);
  // code words [t][slice], params [slice] of chunk q
  auto load_chunk = [&](int q, uint32_t (&cw)[2][B], uint32_t (&pw)[B]) {
    const uint32_t kb = uint32_t(q >> 2) * kTileBytes + 4u * (q & 3), g = uint32_t(q >> a.gshift) * 64u;
#pragma unroll
    for (int j = 0; j < B; ++j) {
      cw[0][j] = __builtin_amdgcn_raw_buffer_load_b32(rs[j], code_voff, kb, 0);
      cw[1][j] = __builtin_amdgcn_raw_buffer_load_b32(rs[j], code_voff, kb + 256u, 0);
      pw[j] = __builtin_amdgcn_raw_buffer_load_b32(rs[j], par_voff, g, 0);
    }
  };

  // ---- activations: chunks of 64 inputs, rows of 128 bytes in LDS.  The 16-byte piece
  // p of row t sits at piece p ^ sw(t), sw(t) = (t & 7) ^ ((t >> 3) & 1): an MFMA operand
  // read (16 consecutive rows, one piece) then covers all 64 banks once, and any 8
  // consecutive rows hit distinct 16-byte bank groups.  Two buffers: chunk q is read
  // while q + 1 is written from registers loaded during q - 1.  Rows past the tile's
  // tokens repeat its last token (never stored).
  const __amdgpu_buffer_rsrc_t xrs = rsrc(a.x, a.x_bytes);
  constexpr int NP = XBF16 ? BM / 64 : BM / 32;  // 16-byte loads per thread and chunk
  constexpr uint32_t XCH = XBF16 ? 128u : 256u;  // bytes of x per row and chunk
  uint32_t xoff[NP], soff[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    // bf16: thread -> (row tid / 8 + 64 p, piece tid % 8); float32: (row tid / 16 + 32 p,
    // four inputs tid % 16, written as half a piece)
    const int t = XBF16 ? (tid >> 3) + 64 * p : (tid >> 4) + 32 * p;
    const int pc = XBF16 ? (tid & 7) : (tid & 15);
    xoff[p] = uint32_t(a.perm[start + min(t, rows - 1)]) * a.x_row + 16u * pc;
    const int sw = (t & 7) ^ ((t >> 3) & 1);
    soff[p] = XBF16 ? 128u * t + 16u * (pc ^ sw)
                    : 128u * t + 16u * ((pc >> 1) ^ sw) + 8u * (pc & 1);
  }
  u32x4_t R[NP];
  auto stage_load = [&](int p, int q) {
    R[p] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff[p], uint32_t(q) * XCH, 0));
  };
  auto stage_write = [&](int p, uint8_t* buf) {
    if constexpr (XBF16) {
      *reinterpret_cast<u32x4_t*>(buf + soff[p]) = R[p];
    } else {
      typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
      const f32x4_t v = __builtin_bit_cast(f32x4_t, R[p]);
      *reinterpret_cast<u32x2_t*>(buf + soff[p]) = u32x2_t{pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3])};
    }
  };

  // the exponent patterns live in vector registers (an AND-OR takes one scalar operand)
  Magic mg;
  asm("v_mov_b32 %0, 0x64006400" : "=v"(mg.m[0]));
  asm("v_mov_b32 %0, 0x5c005c00" : "=v"(mg.m[1]));
  asm("v_mov_b32 %0, 0x54005400" : "=v"(mg.m[2]));
  asm("v_mov_b32 %0, 0x4c004c00" : "=v"(mg.m[3]));

  f32x16_t acc[MB][2];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int k = 0; k < 2; ++k) acc[i][k] = f32x16_t{};

  // A operand of step s, block i: row WM wm + 32 i + col, logical piece 4 c2 + s
  // (sw of the row depends on its low 4 bits only, i.e. on col)
  const uint32_t a_base = 128u * (WM * wm + col) + 16u * ((4 * c2) ^ (col & 7) ^ ((col >> 3) & 1));
  auto abuf = [&](int q) { return lds + (q & 1) * ABUF; };
  auto bx = [&](int q, int k, int s) {   // B operand (column half k, step s) of chunk q
    return lds + BX + (q & 1) * 32768 + ((wn * 2 + k) * 4 + s) * 1024 + 16 * lane;
  };

  uint32_t cw0[2][B], pw0[B], cw1[2][B], pw1[B];
  Consts<B> K;
  const int NQ = a.NQ;

  // ---- dequantization of one chunk's column half: 4 steps x 4 bf16 pairs, pair f of
  // step sp written to the exchange buffer once complete
  Prep<B> P;
  u32x4_t bnew;

  // ---- prologue: chunk 0's activations and weights in LDS, chunk 1 in registers
#pragma unroll
  for (int p = 0; p < NP; ++p) stage_load(p, 0);
  load_chunk(0, cw0, pw0);
#pragma unroll
  for (int p = 0; p < NP; ++p) stage_write(p, abuf(0));
#pragma unroll
  for (int p = 0; p < NP; ++p) stage_load(p, min(1, NQ - 1));
  load_chunk(min(1, NQ - 1), cw1, pw1);
  K = consts<B>(pw0);
#pragma unroll
  for (int sp = 0; sp < 4; ++sp) {
    P = (sp & 1) ? prep<B, 1>(cw0[sp >> 1]) : prep<B, 0>(cw0[sp >> 1]);
#pragma unroll
    for (int f = 0; f < 4; ++f) bnew[f] = pair<B>(P, K, mg, f);
    *reinterpret_cast<u32x4_t*>(bx(0, wm, sp)) = bnew;
  }
  __syncthreads();

  // One chunk q = 4 MFMA steps x MB row blocks = 4 MB groups.  Group g of step s:
  //   MFMA(column half 0) | first halves of the group's bf16 pairs of chunk q + 1 |
  //   MFMA(column half 1) | second halves
  // fenced so that the VALU work sits between the MFMAs (the SIMD's other wave fills the
  // rest).  A operands are read two groups ahead, B operands one step ahead.  The first
  // groups move chunk q + 1's activations to LDS and start loading q + 2's; the codes of
  // q + 2 load into the slot that chunk q's used.
  constexpr int NG = 4 * MB, PPG = 16 / NG;   // groups per chunk, bf16 pairs per group
  auto body = [&](int q, uint32_t (&cwn)[2][B], uint32_t (&pwn)[B], uint32_t (&cwl)[2][B],
                  uint32_t (&pwl)[B]) {
    const uint8_t* cur = abuf(q);
    uint8_t* nxt = abuf(q + 1);
    const int q2 = min(q + 2, NQ - 1);
    K = consts<B>(pwn);
    load_chunk(q2, cwl, pwl);
    auto a_rd = [&](int g) {
      return *reinterpret_cast<const u32x4_t*>(cur + (a_base ^ (16u * (g / MB))) + (g % MB) * 4096);
    };
    u32x4_t av[NG], bv[4][2];
    av[0] = a_rd(0);
    av[1] = a_rd(1);
#pragma unroll
    for (int k = 0; k < 2; ++k) bv[0][k] = *reinterpret_cast<const u32x4_t*>(bx(q, k, 0));
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int s = g / MB, i = g % MB;
      if (g + 2 < NG) av[g + 2] = a_rd(g + 2);
      if (i == 0 && s < 3) {
#pragma unroll
        for (int k = 0; k < 2; ++k) bv[s + 1][k] = *reinterpret_cast<const u32x4_t*>(bx(q, k, s + 1));
      }
      acc[i][0] = mfma32(av[g], bv[s][0], acc[i][0]);
      __builtin_amdgcn_sched_barrier(0);
      Half<B> hv[PPG];
#pragma unroll
      for (int e = 0; e < PPG; ++e) {
        const int pi = g * PPG + e, sp = pi >> 2, f = pi & 3;
        if (f == 0) P = (sp & 1) ? prep<B, 1>(cwn[sp >> 1]) : prep<B, 0>(cwn[sp >> 1]);
        hv[e] = pair_a<B>(P, K, mg, f);
        // keep the first half here: without a use before the fence, the compiler sinks
        // it next to the second half, behind the second MFMA
        asm volatile("" : "+v"(hv[e].lo));
      }
      if (g < NP) {
        stage_write(g, nxt);
        stage_load(g, q2);
      }
      __builtin_amdgcn_sched_barrier(0);
      acc[i][1] = mfma32(av[g], bv[s][1], acc[i][1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int e = 0; e < PPG; ++e) {
        const int pi = g * PPG + e, sp = pi >> 2, f = pi & 3;
        bnew[f] = pair_b<B>(hv[e], K, f);
        // (past the last chunk this rewrites the clamped chunk into the idle buffer)
        if (f == 3) *reinterpret_cast<u32x4_t*>(bx(q + 1, wm, sp)) = bnew;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  };

  int q = 0;
  for (; q + 1 < NQ; q += 2) {
    body(q, cw1, pw1, cw0, pw0);
    body(q + 1, cw0, pw0, cw1, pw1);
  }
  if (q < NQ) body(q, cw1, pw1, cw0, pw0);

  // ---- low-rank side path: acc += u . B^T, 16 ranks per MFMA step, u as a bf16 hi + lo
  // pair.  MFMA k group c2 is ranks k0 + 8 c2 .. + 7 on both operands: the A rows are the
  // tile's tokens (row -> token table; padding rows read zeros), the B columns its outputs.
  if (a.lr_r > 0) {
    const int R = a.lr_r;
    const __amdgpu_buffer_rsrc_t ru = rsrc(a.lr_u, uint32_t(a.lr_ks) * uint32_t(a.T) * uint32_t(R) * 4u);
    const __amdgpu_buffer_rsrc_t rb = rsrc(a.lr_b, uint32_t(a.N) * uint32_t(R) * 2u);
    for (int k0 = 0; k0 < R; k0 += 16) {
      const int kk = k0 + 8 * c2;
      u32x4_t bl[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int n = n0 + 64 * wn + 32 * k + col;
        const uint32_t off = (kk < R && n < a.N) ? (uint32_t(n) * R + kk) * 2u : 0x80000000u;
        bl[k] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0));
      }
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int tok = tokT[WM * wm + 32 * i + col];
        f32x4_t f0{0.f, 0.f, 0.f, 0.f}, f1{0.f, 0.f, 0.f, 0.f};
        for (int z = 0; z < a.lr_ks; ++z) {
          const uint32_t off = (tok >= 0 && kk < R) ? ((uint32_t(z) * a.T + tok) * R + kk) * 4u : 0x80000000u;
          f0 += __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ru, off, 0, 0));
          f1 += __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                    ru, off == 0x80000000u ? off : off + 16u, 0, 0));
        }
        const u32x4_t u0 = __builtin_bit_cast(u32x4_t, f0), u1 = __builtin_bit_cast(u32x4_t, f1);
        u32x4_t uh, ul;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float v0 = __uint_as_float(d < 2 ? u0[2 * d] : u1[2 * d - 4]);
          const float v1 = __uint_as_float(d < 2 ? u0[2 * d + 1] : u1[2 * d - 3]);
          const uint32_t h0 = bf16_bits_rne(v0), h1 = bf16_bits_rne(v1);
          uh[d] = h0 | (h1 << 16);
          ul[d] = bf16_bits_rne(v0 - bf16_bits_to_float(h0)) | (bf16_bits_rne(v1 - bf16_bits_to_float(h1)) << 16);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          acc[i][k] = mfma32(uh, bl[k], acc[i][k]);
          acc[i][k] = mfma32(ul, bl[k], acc[i][k]);
        }
      }
    }
  }

  if (a.y_bf16)
    store_tile<MB, WM, true>(acc, a, tokT, lds, wave, wn, wm, lane, n0);
  else
    store_tile<MB, WM, false>(acc, a, tokT, lds, wave, wn, wm, lane, n0);
}

// Tiles.  A budget group of R tokens takes R / BMb full tiles of BMb tokens (256; 128
// for float32 activations); a remainder of more than half a tile takes one more full
// tile, a smaller one (bf16 activations) a half tile of 128 tokens, so the padding stays
// below half a tile.  All full tiles are numbered first, then the half tiles, each as
// (M tile, N tile) with N fastest, and tile i runs on workgroup i.  Workgroups are dealt
// to the eight XCDs round-robin and, within an XCD, dispatched in order, so every XCD
// starts its share of full tiles and fills the tail with half tiles (a longest-first
// schedule); the grid is sized for the most tiles any budget split can need and the real
// count comes from offsets.  The 256 MiB last-level cache serves the activation and
// weight tiles that several XCDs read.
//
// One workgroup fills a CU (its LDS), so P workgroups run at once (P = the CU count).
// When the full tiles outnumber P, the F - P of them past the first round would make a
// second round as long as the first while most CUs idle.  If halving them (two tiles of
// 128 tokens each, numbered right after the first P) lets the second round's tiles, the
// budget groups' own half tiles included, fit in P, they are halved: the second round
// then takes a half tile's time (the dequantization of 256 outputs plus half the MFMAs).
template <bool XBF16>
__global__ __launch_bounds__(512) void prefill_mfma_kernel(TileArgs a, int S, int P,
                                                           const int32_t* __restrict__ offsets) {
  constexpr int BMb = XBF16 ? 256 : 128, BMs = XBF16 ? 128 : 0;
  __shared__ __attribute__((aligned(16))) uint8_t lds[lds_bytes<XBF16>()];
  const int T = a.T;
  int lo_[5] = {}, hi_[5] = {}, full_[5] = {}, half_[5] = {}, nfull = 0, nhalf = 0;
  // (loops over the at most 4 budget groups are unrolled so the tables stay in registers)
#pragma unroll
  for (int bb = 1; bb <= 4; ++bb) {
    if (bb > S) break;
    // offsets out of contract are clamped into [0, T] so no tile reaches past perm
    const int lo = min(max(offsets[bb - 1], 0), T), hi = min(max(offsets[bb], lo), T);
    const int R = hi - lo, rem = R % BMb;
    lo_[bb] = lo;
    hi_[bb] = hi;
    half_[bb] = (BMs > 0 && rem > 0 && rem <= BMs) ? 1 : 0;
    full_[bb] = R / BMb + ((rem > 0 && !half_[bb]) ? 1 : 0);
    nfull += full_[bb];
    nhalf += half_[bb];
  }
  const int NT = (a.N + kBN - 1) / kBN;
  // tile ti in the unsplit numbering (full tiles, then half tiles) and, for a halved full
  // tile, which 128 of its tokens (part 0 or 1)
  const int F = NT * nfull, H = NT * nhalf;
  const int X = (BMs > 0 && F > P && 2 * (F - P) + H <= P) ? F - P : 0;
  const int lin = blockIdx.x;
  int ti = lin, part = -1;
  if (X > 0 && lin >= P) {
    if (lin < P + 2 * X) {
      ti = P + ((lin - P) >> 1);
      part = (lin - P) & 1;
    } else {
      ti = lin - X;
    }
  }
  if (ti >= F + H) return;
  int m = ti / NT;
  const int n0 = (ti % NT) * kBN;
  bool is_half = m >= nfull;
  if (is_half) m -= nfull;
  int b = 0, start = 0, rows = 0;
#pragma unroll
  for (int bb = 1; bb <= 4; ++bb) {
    if (bb > S) break;
    const int cnt = is_half ? half_[bb] : full_[bb];
    if (m < cnt) {
      b = bb;
      start = is_half ? lo_[bb] + (full_[bb] * BMb) : lo_[bb] + m * BMb;
      rows = min(is_half ? BMs : BMb, hi_[bb] - start);
      break;
    }
    m -= cnt;
  }
  if (b == 0) return;  // uniform; unreachable for lin below the tile count
  if (part >= 0) {
    // a full tile holds more than BMs rows, so either part has at least one
    start += BMs * part;
    rows = min(BMs, rows - BMs * part);
    is_half = true;
  }
  if constexpr (BMs > 0) {
    if (is_half) {
      switch (b) {
        case 1: prefill_tile<1, XBF16, BMs>(a, start, rows, n0, lds); break;
        case 2: prefill_tile<2, XBF16, BMs>(a, start, rows, n0, lds); break;
        case 3: prefill_tile<3, XBF16, BMs>(a, start, rows, n0, lds); break;
        default: prefill_tile<4, XBF16, BMs>(a, start, rows, n0, lds); break;
      }
      return;
    }
  }
  switch (b) {
    case 1: prefill_tile<1, XBF16, BMb>(a, start, rows, n0, lds); break;
    case 2: prefill_tile<2, XBF16, BMb>(a, start, rows, n0, lds); break;
    case 3: prefill_tile<3, XBF16, BMb>(a, start, rows, n0, lds); break;
    default: prefill_tile<4, XBF16, BMb>(a, start, rows, n0, lds); break;
  }
}

// Workgroups of the kernel that run at once: one per CU, unless the caller states a count
// (it only changes which full tiles are halved, never the results' definition).
int resident_slots(int32_t slots) {
  if (slots > 0) return slots;
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

}  // namespace

bool prefill_mfma_supported(const mbq_desc& d, int32_t t, const void* x, bool x_bf16) {
  const uint64_t x_bytes = uint64_t(t) * d.k * (x_bf16 ? 2 : 4);
  // groups of 32 inputs are served by the generic kernel
  return t > 0 && d.group >= 64 && d.slice_stride < (1ull << 32) && x_bytes < (1ull << 32) &&
         (reinterpret_cast<uintptr_t>(x) & 15) == 0;
}

hipError_t launch_prefill_mfma(const mbq_desc& d, const void* packed, int32_t t, const void* x,
                               bool x_bf16, const int32_t* perm, const int32_t* offsets, void* y,
                               bool y_bf16, const float* lr_u, int32_t lr_ks, const uint16_t* lr_b,
                               int32_t lr_r, int32_t slots, hipStream_t stream) {
  const int BM = x_bf16 ? 256 : 128;
  TileArgs a{};
  a.packed = static_cast<const uint8_t*>(packed);
  a.ss = uint32_t(d.slice_stride);
  a.po = uint32_t(d.params_offset);
  a.N = d.n;
  a.KB = d.k_tiles;
  a.NG = d.groups_padded;
  a.NB = d.row_blocks;
  a.gshift = d.group == 64 ? 0 : (d.group == 128 ? 1 : 2);
  a.NQ = d.k / 64;
  a.T = t;
  a.x = x;
  a.x_row = uint32_t(d.k) * (x_bf16 ? 2u : 4u);
  a.x_bytes = uint32_t(uint64_t(t) * a.x_row);
  a.perm = perm;
  a.y = y;
  a.y_bf16 = int(y_bf16);
  a.lr_u = lr_u;
  a.lr_b = lr_b;
  a.lr_r = lr_r;
  a.lr_ks = lr_ks;
  const int NT = (d.n + kBN - 1) / kBN;
  // at most ceil(R / BM) tiles per budget group (a half tile replaces a full one), plus
  // the halved ones: at most P / 2, since halving requires 2 (F - P) + H <= P
  const int P = resident_slots(slots);
  const int max_tiles = NT * ((t + BM - 1) / BM + d.slices - 1) + P / 2;
  dim3 grid(max_tiles), block(512);
  if (x_bf16)
    hipLaunchKernelGGL(prefill_mfma_kernel<true>, grid, block, 0, stream, a, d.slices, P, offsets);
  else
    hipLaunchKernelGGL(prefill_mfma_kernel<false>, grid, block, 0, stream, a, d.slices, P, offsets);
  return hipGetLastError();
}

}  // namespace mbq
