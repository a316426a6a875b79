// Routed decode linear for small batches (T <= 64) -- the HBM-streaming kernel.
//
// Same arithmetic as decode.hip (MoBiQuant explainer, gist.science English page, sections
// 2.A and 3: each token sums its own slices; only slices some token uses are fetched):
//   y[t, n] = sum_j [b(t) >= j] sum_g ( s_jng * P_jng[t] + z_jng * X_g[t] ),
//   P = sum_{k in g} x_k q_k, on one of two multiplies:
//   * bf16 operands: MFMA 16x16x32 bf16 with raw codes as bf16 (o + q) values and the
//     accumulator seeded with -sum_k x_k o_k;
//   * F4: MFMA 16x16x128 fp8 x fp4 with the codes as e2m1 nibbles (q / 2, B scale 2) and the
//     activations split exactly into e4m3 hi + lo pairs (see the F4 section below).
//
// Organisation (one persistent workgroup per CU):
//   * tokens come in blocks of 16 (workgroup row blockIdx.y, at most 4 for T <= 64), one
//     MFMA token block each; rows stay in the tokens' original order, so x is read with no
//     dependence on perm, and perm / offsets only decide which slices count for which row;
//   * wave w owns k tiles w, w + NW, ... (TPW of them): their slice of its token block's x
//     (the A operand) and the per-group seeds -sum x*o and sums X are computed once and stay
//     in registers (X in LDS) for the whole kernel;
//   * the workgroup walks row blocks nb = blockIdx.x, + gridDim.x, ...; for each, every
//     wave multiplies its k tiles of every needed slice while the next two row blocks'
//     codes and params are already loading (three register buffers with fixed roles,
//     every load unconditional: a past-the-end row block re-reads cached lines, a slice no
//     token of the batch uses has an empty buffer range and reads nothing);
//   * the waves' partial 16x16 tiles are summed in LDS (double-buffered, one barrier per
//     row block) and written out with per-token slice masks already applied.
// Token perm[i] (sorted position i) has budget b with offsets[b-1] <= i < offsets[b].
// With RT (the one-launch decode step, mbq_route_linear) the kernel computes perm and
// offsets itself: see RouteIO below.
#include <type_traits>

#include "mbq_internal.h"

namespace mbq {
namespace {

constexpr int kMaxWaves = 8;
// In-kernel routing: batches of at most this many tokens issue row block 1's second and
// later slices only once the budgets are known, with the slices some token uses (a
// one-token step usually reads one of three slices, and those loads, issued earlier,
// stalled the routing behind the memory queue); its first slice, which every token uses,
// goes out with row block 0.
constexpr int kLateRow1 = 1;
constexpr int kMaxTokens = 64;  // tokens per launch (16 per workgroup row)
// Reads of u (side path with lr_fz) before giving up: each is a round trip to memory plus
// a short sleep, so this bounds the wait at about a tenth of a second.
constexpr int kLrSpin = 1 << 16;
// Variants that carry the in-launch u (lr_fz): all but float32 activations over two k
// tiles per wave, whose registers are full without it.
constexpr bool lr_inline_fits(int NA, int TPW) { return !(NA == 2 && TPW == 2); }
// Row blocks per workgroup whose float32 sums LDS can hold until the side path is added
// (LR with lr_fz; 1 KiB each).  The host computes u in a launch of its own beyond this.
constexpr int kLrStage = 48;
constexpr uint32_t kNeg128 = 0xC300C300u, kNeg32 = 0xC200C200u, kNeg8 = 0xC100C100u;
constexpr uint32_t kOnes = 0x3F803F80u;

// Masks in scalar registers and the bf16 exponent patterns in vector registers, so that
// (a & mask) | magic is one v_and_or_b32 (gfx9 VOP3 takes no literal constants and reads
// at most one scalar operand).  Plain C: the compiler sees every producer of an MFMA
// operand and inserts whatever wait states the hardware needs.
struct Magic {
  uint32_t m128, m32, m8;  // bf16 pairs 128, 32 and 8 (vector registers)
  uint32_t k3, kc, k30;    // field masks 0x00030003, 0x000C000C, 0x00300030 (scalar registers)
};

__device__ __forceinline__ Magic make_magic() {
  Magic mg{0x43004300u, 0x42004200u, 0x41004100u, 0u, 0u, 0u};
  // keep the patterns in vector registers (as constants they would compete with the mask
  // for the one scalar operand and split every AND-OR in two)
  asm volatile("" : "+v"(mg.m128), "+v"(mg.m32), "+v"(mg.m8));
  mg.k3 = __builtin_amdgcn_readfirstlane(0x00030003u);
  mg.kc = __builtin_amdgcn_readfirstlane(0x000C000Cu);
  mg.k30 = __builtin_amdgcn_readfirstlane(0x00300030u);
  return mg;
}

__device__ __forceinline__ void unpack_word(uint32_t w, const Magic& mg, u32x4_t& b0, u32x4_t& b1) {
  const uint32_t w6 = w >> 6, w12 = w >> 12;
  b0[0] = (w & mg.k3) | mg.m128;     // 128 + q: inputs 0, 1
  b0[1] = (w & mg.kc) | mg.m32;      //  32 + q: inputs 2, 3
  b0[2] = (w & mg.k30) | mg.m8;      //   8 + q: inputs 4, 5
  b0[3] = (w6 & mg.k3) | mg.m128;    // 128 + q: inputs 6, 7
  b1[0] = (w6 & mg.kc) | mg.m32;     //  32 + q: inputs 8, 9
  b1[1] = (w6 & mg.k30) | mg.m8;     //   8 + q: inputs 10, 11
  b1[2] = (w12 & mg.k3) | mg.m128;   // 128 + q: inputs 12, 13
  b1[3] = (w12 & mg.kc) | mg.m32;    //  32 + q: inputs 14, 15
}

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Each MFMA chain is followed by a scheduling fence before its results are read: it keeps
// the compiler from interleaving the next group's chains with this group's epilogue,
// which would lengthen live ranges past the 256 registers of a wave and spill.
__device__ __forceinline__ void chain_fence() { __builtin_amdgcn_sched_barrier(0); }

// ---- F4: bfloat16 activations on the scaled fp8 x fp4 matrix instruction
// (v_mfma_scale_f32_16x16x128_f8f6f4), which takes the codes almost as stored.
//
// A 2-bit code q in the low two bits of a nibble whose upper bits are zero is the e2m1
// (fp4) number q / 2 exactly (0 and 0.5 subnormal, 1 and 1.5 normal), so a code word
// masked with 0x33333333 is eight fp4 values (its codes at bit positions 0, 4, ..., 28:
// inputs 0, 4, 8, 12, 1, 5, 9, 13 of the word's 16) and the word shifted right by two is
// the other eight (inputs 2, 6, 10, 14, 3, 7, 11, 15): three instructions per word where
// bf16 operands take ten.
//
// Operand layouts of the instruction (16 x 16 x 128, measured on gfx950): byte q of lane
// (r, c)'s A operand (8 registers of e4m3) is row r, logical input 16c + (q mod 16) +
// 64 (q div 16); nibble p of lane (n, c)'s B operand (4 registers of e2m1) is column n,
// logical input 32c + p; the e8m0 scale of row r (column n) and logical inputs 32b ..
// 32b + 31 comes from lane r + 16b (n + 16b).  B of lane (n, c) is its code words 2m and
// 2m + 1 of the tile (inputs 128m + 64 i' + 16c + e, i' = 0, 1), masked even and odd, which
// makes logical input 32c + 8j + t the physical input 128m + 64 (j >> 1) + 16c +
// E_(j & 1)(t), E_0 = (0 4 8 12 1 5 9 13), E_1 = (2 6 10 14 3 7 11 15).  The A operand is
// loaded to match: lane (r, c) holds token r's inputs 128m + 64 (c & 1) + 16 (c >> 1) +
// [0, 16) and the same + 32, bytes in the order E_0, E_1 within each run.
//
// The activations of a 128-input block are split exactly into two e4m3 numbers with one
// power-of-two scale per token row: sc = 2^(e8 - 127) puts the row's largest |x| of the
// 128 in [128, 256) sc, hi = e4m3(x / sc) and lo = e4m3((x - hi sc) / sc), both rounded to
// nearest even (the scaled converters of gfx950); hi + lo = x / sc exactly for every
// |x / sc| >= 1/4 (2^-10 of the block's largest), smaller inputs keep an absolute error
// below 2^-10 sc.  The instruction's own sum of the 128 products is not exact: measured,
// its error is about 1e-5 of the sum of |products|.
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((ext_vector_type(2))) short i16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

struct AF4 {
  i32x8_t hi, lo;
  uint32_t sc;  // e8m0 scale of the lane's row (every lane of a row holds the same)
};

__device__ __forceinline__ uint32_t f4_even(uint32_t w) { return w & 0x33333333u; }
__device__ __forceinline__ uint32_t f4_odd(uint32_t w) { return (w >> 2) & 0x33333333u; }

// B's scale is 2 (e8m0 128) for code products, so they come out as sum x q, and 1 (127)
// for the group sums, whose B operand is every nibble 1.0
template <int BSCALE>
__device__ __forceinline__ f32x4_t mfma_f4(const i32x8_t& a, const uint32_t (&bw)[4], uint32_t scale, f32x4_t c) {
  const i32x8_t b{int(bw[0]), int(bw[1]), int(bw[2]), int(bw[3]), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, int(scale), 0, BSCALE);
}

// One byte pair (q, q + 1) of the hi and lo registers: x0, x1 in float32 (word half sel).
template <bool SEL>
__device__ __forceinline__ void split_pair(float x0, float x1, float sc, int& hw, int& lw) {
  i16x2_t h = __builtin_bit_cast(i16x2_t, hw), l = __builtin_bit_cast(i16x2_t, lw);
  h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h, x0, x1, sc, SEL);
  const f32x2_t hb = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(__builtin_bit_cast(int, h), sc, SEL);
  l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l, x0 - hb[0], x1 - hb[1], sc, SEL);
  hw = __builtin_bit_cast(int, h);
  lw = __builtin_bit_cast(int, l);
}

// run[0], run[1]: inputs base + [0, 16) of the lane's token (8 bf16 each); run[2], run[3]:
// base + 32 + [0, 16).  Every lane of the wave takes part (the row maximum crosses lanes).
__device__ __forceinline__ AF4 prep_a_f4(const u32x4_t& r0, const u32x4_t& r1, const u32x4_t& r2,
                                         const u32x4_t& r3) {
  const u32x4_t run[4] = {r0, r1, r2, r3};
  float v[32];
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      v[8 * h + 2 * d] = __uint_as_float(run[h][d] << 16);
      v[8 * h + 2 * d + 1] = __uint_as_float(run[h][d] & 0xFFFF0000u);
    }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  // e8 >= 1 keeps the scale a normal float (rows below 2^-119 lose their small bits)
  const int e8 = max(int(__float_as_uint(m) >> 23) - 7, 1);
  const float sc = __uint_as_float(uint32_t(e8) << 23);
  constexpr int kE[16] = {0, 4, 8, 12, 1, 5, 9, 13, 2, 6, 10, 14, 3, 7, 11, 15};
  AF4 a;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = 4 * j;  // bytes q .. q + 3: run q >> 4, elements kE[(q & 15) ..]
    const float* vr = &v[16 * (q >> 4)];
    int hw = 0, lw = 0;
    split_pair<false>(vr[kE[q & 15]], vr[kE[(q & 15) + 1]], sc, hw, lw);
    split_pair<true>(vr[kE[(q & 15) + 2]], vr[kE[(q & 15) + 3]], sc, hw, lw);
    a.hi[j] = hw;
    a.lo[j] = lw;
  }
  a.sc = uint32_t(e8);
  return a;
}

// Two floats rounded to nearest even into one register of two bfloat16 (a low, b high):
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

__device__ __forceinline__ u32x4_t ldg16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// The low-rank side path's B rows of one row block travel with its codes (LR only).
template <bool LR>
struct LrRows {
  u32x4_t v;
};
template <>
struct LrRows<false> {};

// One row block's loads for one wave: its tiles' code words and, per slice, the float16
// (scale, zero) pairs of its NE (tile, group) units with one 4-byte load per 64 lanes:
// lane 16 q + r of pw[j][h] holds unit 4 h + q of row r (spread to every lane of the
// row by bcast_rows before use), instead of one load per unit.
template <int G, int S, int TPW, bool LR = false>
struct Codes {
  static constexpr int GPT = 256 / G, NE = TPW * GPT, PH = (NE + 3) / 4;
  u32x4_t cw[TPW][S];
  uint32_t pw[S][PH];
  LrRows<LR> lr;
};

// Row q (lanes 16 q .. 16 q + 15) of v copied to every row, for q = 0 .. 3: one swap of
// the wave's halves and two of alternate rows (gfx950 v_permlane32_swap /
// v_permlane16_swap).
__device__ __forceinline__ void bcast_rows(uint32_t v, uint32_t (&o)[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);        // rows 0 1 0 1 | 2 3 2 3
  const auto b = __builtin_amdgcn_permlane16_swap(a[0], a[0], false, false);  // rows 0 0 0 0 | 1 1 1 1
  const auto c = __builtin_amdgcn_permlane16_swap(a[1], a[1], false, false);  // rows 2 2 2 2 | 3 3 3 3
  o[0] = b[0];
  o[1] = b[1];
  o[2] = c[0];
  o[3] = c[1];
}

// Raw buffer loads: one scalar resource per slice, a scalar tile offset and one per-lane
// offset that never changes, so the loop needs no vector address arithmetic.  (Buffer
// loads are also bounds-checked by the hardware against the slice size.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const uint8_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, int(bytes), 0x00020000);
}

// lane_pv[h]: the lane's byte offset of unit 4 h + (lane >> 4), row lane & 15, within a
// row block's params (past the slice for units the wave does not have).
template <int G, int S, int TPW, bool LR>
__device__ __forceinline__ void load_codes(Codes<G, S, TPW, LR>& C, const __amdgpu_buffer_rsrc_t (&rs)[S],
                                           int nb, const int (&kt)[TPW], int KB, int NG,
                                           uint32_t po, uint32_t lane_code,
                                           const uint32_t (&lane_pv)[Codes<G, S, TPW, LR>::PH],
                                           int jlo = 0, int jhi = S) {
  // (slices [jlo, jhi) only: the callers pass constants, so the loop below stays unrolled)
  constexpr int PH = Codes<G, S, TPW, LR>::PH;
  // nb < 0: a row block past the workgroup's last one.  Its loads still go out (every
  // path keeps the same loads in flight) but at an offset past every buffer's range
  // (slices end below 2^32 - 256), so they return zeros without a memory request.
  const bool dead = nb < 0;
  constexpr uint32_t kPastEnd = 0xFFFFFFF0u;
  const uint32_t vc = dead ? kPastEnd : lane_code;
#pragma unroll
  for (int j = 0; j < S; ++j) {
    if (j < jlo || j >= jhi) continue;
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp) {
      const uint32_t tile = dead ? 0u : uint32_t(nb * KB + kt[tp]) * kTileBytes;
      C.cw[tp][j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs[j], vc, tile, 0));
    }
    const uint32_t par = dead ? 0u : po + uint32_t(nb * NG) * 64;
#pragma unroll
    for (int h = 0; h < PH; ++h)
      C.pw[j][h] = __builtin_amdgcn_raw_buffer_load_b32(rs[j], dead ? kPastEnd : lane_pv[h], par, 0);
  }
}

// At most 8 waves (two per SIMD), so a wave has 256 registers: room for its stationary
// A operand and seeds plus three buffers of codes and params without any spill (a spill
// would wait on the in-order load counter behind the prefetched loads).
//
// LR adds the low-rank side path u_t . B^T (u = x A^T from lowrank.hip, [T x R] float32;
// B [N x R] bf16, R a multiple of 8 up to 32): wave 0 of the first k chunk multiplies the
// token block's u (a bf16 hi + lo pair, held for the whole launch) by the row block's B
// rows (loaded with its codes) in two more MFMAs and adds the product to its part of the
// output before the waves' parts are summed.
// RT routes the batch inside the kernel (MoBiRoute, linear-argmax form, and the regroup:
// MoBiQuant explainer, gist.science English page, section 2.B) instead of reading perm
// and offsets: T <= 16 tokens (one token block), K within one workgroup.  Every wave
// takes the dot products of its own activations (already in registers) with Wr rows
// staged in LDS; the lanes' and waves' partial sums are added in a fixed order, so every
// workgroup derives bit-identical logits and budgets, and workgroup 0 writes logits,
// budget, perm and offsets for the caller.
struct RouteIO {
  const float* wr;  // [K x S] row-major
  float* logits;    // [T x S]
  int32_t* budget;  // [T]
  int32_t* perm;    // [T]
  int32_t* offsets; // [S + 1]
  const uint8_t* prep;  // PA: decode_prep_kernel's output (layout: PrepLayout)
};

// The prepared activations of one decode step (PA; written by decode_prep_kernel, one
// record per k tile of 256 inputs, 16 tokens): the fp8 x fp4 multiply's A operands as
// register images (8 chunks of 64 lanes x 16 bytes: e4m3 hi of block 0, lo of block 0, hi
// of block 1, lo of block 1, two chunks each), their e8m0 scales (64 lanes x 2 words),
// the per-group activation sums (GPT x 16 floats) and the tile's partial router logits
// (16 tokens x 4 floats).  Sections are contiguous over the k tiles.
struct PrepLayout {
  uint32_t a, sc, xs, lg, bytes;
  __host__ __device__ PrepLayout(int KB, int G) {
    a = 0;
    sc = a + uint32_t(KB) * 8192u;
    xs = sc + uint32_t(KB) * 512u;
    lg = xs + uint32_t(KB) * uint32_t(256 / G) * 64u;
    bytes = lg + uint32_t(KB) * 256u;
  }
};

template <int G, int S, int NA, int TPW, int TB, bool LR, bool RT, bool F4, bool PA = false>
__global__ __launch_bounds__(512) void decode_stream_kernel(
    const uint8_t* __restrict__ packed, int N, int K, int KB, int NG, int NB, uint64_t ss,
    uint64_t po, const void* __restrict__ x, int T, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, void* __restrict__ y, int y_bf16, int kchunk,
    float* __restrict__ part, const float* __restrict__ lr_u, int lr_ks,
    const uint16_t* __restrict__ lr_b, int lr_r, uint8_t* __restrict__ lr_fz,
    const uint16_t* __restrict__ lr_a, RouteIO rio) {
  static_assert(!LR || TB == 1, "the side path is built for one token block per workgroup");
  static_assert(!RT || (TB == 1 && !LR), "in-kernel routing takes one token block, no side path");
  static_assert(!F4 || (NA == 1 && TB == 1 && !LR), "fp4 operands: bfloat16 activations, one token block");
  static_assert(!PA || (RT && F4), "prepared activations: the routed fp8 x fp4 step");
  // Every kernel argument is read in one batch behind one wait: loaded lazily, they come
  // from up to three scalar cache lines in turn, each a round trip before the first
  // activation load can be issued.
  asm volatile("" ::"s"(packed), "s"(x), "s"(perm), "s"(offsets), "s"(y), "s"(part), "s"(lr_u), "s"(lr_b));
  asm volatile("" ::"s"(N), "s"(K), "s"(KB), "s"(NG), "s"(NB), "s"(ss), "s"(po), "s"(T), "s"(y_bf16),
               "s"(kchunk), "s"(lr_ks), "s"(lr_r));
  if constexpr (LR) asm volatile("" ::"s"(lr_fz), "s"(lr_a));
  if constexpr (RT) asm volatile("" ::"s"(rio.wr), "s"(rio.logits), "s"(rio.budget), "s"(rio.perm), "s"(rio.offsets));
  if constexpr (PA) asm volatile("" ::"s"(rio.prep));
  constexpr int GPT = 256 / G, WPG = G / 64;
  __shared__ f32x4_t red[2][kMaxWaves][TB][64];
  const int NW = blockDim.x >> 6;
  // the wave index is uniform: telling the compiler keeps tile addresses in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane & 15, c = lane >> 4;
  // LR with lr_fz: workgroup 0 of each token block computes u itself (see lr_produce)
  // and the others stream the row blocks, so they count from blockIdx.x - 1
  // (not built where the wave's registers are already full: float32 activations over two
  // tiles; the host computes u in a launch of its own there)
  const bool lrf = lr_inline_fits(NA, TPW) && LR && lr_fz != nullptr;
  const int step = lrf ? int(gridDim.x) - 1 : int(gridDim.x);

  // k tiles [kb0, kend) of this workgroup's k chunk (blockIdx.z)
  const int kb0 = blockIdx.z * kchunk, kend = min(KB, kb0 + kchunk);
  int kt[TPW];
  bool live[TPW];
#pragma unroll
  for (int tp = 0; tp < TPW; ++tp) {
    const int t = kb0 + wave + NW * tp;
    live[tp] = t < kend;
    kt[tp] = live[tp] ? t : kb0;
  }

  // ---- 1. routing.  The number of slices read (jmax) comes from offsets alone: 1 +
  // #{j >= 1 : offsets[j] < T} (every slice some token of the batch uses).  offsets[0..S]
  // arrive through one vector load (lane j takes offsets[j]) and are read back with
  // readlane after the activation loads have been issued: a scalar load would sit in front
  // of them, since a wait for any later kernel argument waits for every scalar load.
  // Per-token budgets come from perm: lane i of wave 0 takes sorted position i (T <= 64)
  // and later publishes that token's budget in an LDS table.  Both loads are issued
  // first, so waiting for them never waits for the activation loads behind them.
  const int offv = RT ? 0 : offsets[min(lane, S)];
  const int pi = (!RT && wave == 0 && lane < T) ? perm[lane] : -1;

  // The side path's u rows of this token block: lane (r, c) holds ranks 8c .. 8c + 7 of
  // token row r (clamped like the activations; ranks past R read zeros), summed over the
  // lr_ks chunks of K in order.  Issued before the activations so that the sum waits
  // for these loads only.
  __amdgpu_buffer_rsrc_t rlr_b = slice_rsrc(reinterpret_cast<const uint8_t*>(lr_b), 0u);
  uint32_t lr_lane = 0;
  u32x4_t Uraw[2], Uop[2];
  if constexpr (LR) {
    const int xr = 16 * TB * blockIdx.y + min(r, min(16 * TB, T - 16 * TB * int(blockIdx.y)) - 1);
    const __amdgpu_buffer_rsrc_t ru =
        slice_rsrc(reinterpret_cast<const uint8_t*>(lr_u), uint32_t(lr_ks) * uint32_t(T) * lr_r * 4);
    u32x4_t ul[kMaxLrChunks][2];
#pragma unroll
    for (int z = 0; z < kMaxLrChunks; ++z) {
      const uint32_t uo = (8 * c < lr_r && z < lr_ks) ? ((uint32_t(z) * T + xr) * lr_r + 8 * c) * 4 : 0x80000000u;
      ul[z][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ru, uo, 0, 0));
      ul[z][1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ru, uo == 0x80000000u ? uo : uo + 16, 0, 0));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4_t acc = __builtin_bit_cast(f32x4_t, ul[0][h]);
#pragma unroll
      for (int z = 1; z < kMaxLrChunks; ++z) acc += __builtin_bit_cast(f32x4_t, ul[z][h]);  // + 0 past lr_ks
      Uraw[h] = __builtin_bit_cast(u32x4_t, acc);
    }
    // B rows: only wave 0 of k chunk 0 reads them (the others load zeros, no traffic)
    rlr_b = slice_rsrc(reinterpret_cast<const uint8_t*>(lr_b), (wave == 0 && blockIdx.z == 0) ? uint32_t(N) * lr_r * 2 : 0u);
    lr_lane = 8 * c < lr_r ? (uint32_t(r) * lr_r + 8 * c) * 2 : 0x80000000u;
  }
  // With lr_fz the side path's u comes from this launch's workgroup 0 (lr_produce) instead
  // of lr_u.  lr_fz holds: word 0, the launch count E (one more after every launch);
  // word 2, error flags (bit 0: u never arrived, so the side path was left out; bit 1: not
  // every workgroup checked in); from byte kLrSlots, one 128-byte line per workgroup whose
  // first word it sets to E + 1 once it has read E (separate lines: no two workgroups write
  // one line, and there is no read-modify-write atomic, which serialises in memory while
  // the weights stream); from byte kLrPairs, u of token block y, token t, rank q as the
  // 8-byte pair (E + 1) << 32 | float bits, at ((16 y + t) R + q).
  // A pair is one store and one load at device scope, so a reader that sees this launch's
  // tag sees that store's value; pairs left by an earlier launch carry an older tag.
  uint32_t lrE = 0;
  if constexpr (LR)
    if (lrf) lrE = __hip_atomic_load(reinterpret_cast<uint32_t*>(lr_fz), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- 2. this wave's activations.  Workgroup row blockIdx.y takes the TB 16-token
  // blocks starting at token tb0 = 16 TB blockIdx.y; in block b, MFMA row r is token
  // tb0 + 16 b + r (rows past T repeat a real token and are never stored).
  const int tb0 = 16 * TB * blockIdx.y, Tw = min(16 * TB, T - tb0);
  // first input of activation load (i, h) of tile tp within the tile: bf16 operands take
  // inputs 64i + 16c + 8h; fp8 ones (F4) the runs of 128-input block i >> 1 (see above)
  auto xk = [&](int i, int h) {
    return F4 ? 128 * (i >> 1) + 64 * (c & 1) + 16 * (c >> 1) + 32 * (i & 1) + 8 * h : 64 * i + 16 * c + 8 * h;
  };
  u32x4_t Araw[TB][TPW][4][2][NA];
  auto load_x = [&](int b, int tp) __attribute__((always_inline)) {
    const int xr = tb0 + min(16 * b + r, Tw - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < NA; ++q) {
          // K is a multiple of 64, so these 8 inputs are all real or all padding; padding
          // reads the row's first inputs instead (zeroed with the seeds)
          const int k = kt[tp] * 256 + xk(i, h);
          const int kk = k < K ? k : 0;
          const uint8_t* p = static_cast<const uint8_t*>(x) + (size_t(xr) * K + kk) * (2 * NA) + 16 * q;
          Araw[b][tp][i][h][q] = ldg16(p);
        }
  };
  // RT: each tile's Wr rows (kt * 256 .. + 255: 256 S contiguous floats) as 16-byte loads
  // right behind that tile's activations, so the first tile can be routed while the
  // second one's loads are still arriving (Wr ahead of the activations delays what
  // everything else waits for); rows past K read zeros
  u32x4_t wld[RT ? TPW : 1][RT ? S : 1];
  // PA: the prepared operands of this wave's tiles instead (16-byte loads, 1 KiB of
  // consecutive bytes per instruction); a tile the wave does not have reads zeros
  u32x4_t pa_x[PA ? TPW : 1][8];
  uint32_t pa_sc[PA ? TPW : 1][2], pa_xs[PA ? TPW : 1];
  u32x4_t pa_lg[PA ? TPW : 1];
  if constexpr (PA) {
    const PrepLayout pl(KB, G);
    const __amdgpu_buffer_rsrc_t ra = slice_rsrc(rio.prep + pl.a, pl.sc - pl.a);
    const __amdgpu_buffer_rsrc_t rsc = slice_rsrc(rio.prep + pl.sc, pl.xs - pl.sc);
    const __amdgpu_buffer_rsrc_t rxs = slice_rsrc(rio.prep + pl.xs, pl.lg - pl.xs);
    const __amdgpu_buffer_rsrc_t rlg = slice_rsrc(rio.prep + pl.lg, pl.bytes - pl.lg);
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp) {
      const uint32_t t = uint32_t(kt[tp]), none = 0x80000000u;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        pa_x[tp][q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                          ra, live[tp] ? ((t * 8 + q) * 64 + lane) * 16 : none, 0, 0));
      const auto scv = __builtin_amdgcn_raw_buffer_load_b64(rsc, live[tp] ? (t * 64 + lane) * 8 : none, 0, 0);
      pa_sc[tp][0] = uint32_t(scv[0]);
      pa_sc[tp][1] = uint32_t(scv[1]);
      pa_xs[tp] = __builtin_amdgcn_raw_buffer_load_b32(rxs, live[tp] && lane < 16 * GPT ? (t * GPT * 16 + lane) * 4 : none, 0, 0);
      pa_lg[tp] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                      rlg, live[tp] && lane < 16 ? (t * 16 + lane) * 16 : none, 0, 0));
    }
    // Row blocks 0 and 1 go out once every wave of the workgroup has issued its prepared
    // loads (a barrier on the issue, not the data): the second wave on each SIMD can issue
    // only when the first one's loads return, and codes queued in front of it would delay
    // its operands by another round trip.  Every slice's range: the budgets are not known
    // yet, and slices past jmax add nothing (no budget reaches them).
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  } else if constexpr (RT) {
    const __amdgpu_buffer_rsrc_t rw = slice_rsrc(reinterpret_cast<const uint8_t*>(rio.wr), uint32_t(K) * S * 4);
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp) {
      load_x(0, tp);
#pragma unroll
      for (int q = 0; q < S; ++q)
        wld[tp][q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                         rw, (uint32_t(kt[tp]) * 256 * S + (64 * q + lane) * 4) * 4, 0, 0));
    }
  } else {
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int tp = 0; tp < TPW; ++tp) load_x(b, tp);
  }
  // (the fence keeps every activation load ahead of the wait for offsets)
  __builtin_amdgcn_sched_barrier(0);
  int off[S + 1];
#pragma unroll
  for (int j = 0; j <= S; ++j) off[j] = __builtin_amdgcn_readlane(offv, j);
  int jmax = 1;
#pragma unroll
  for (int j = 1; j < S; ++j)
    if (off[j] <= T - 1) jmax = j + 1;

  auto load_lr = [&](Codes<G, S, TPW, LR>& C, int nb) __attribute__((always_inline)) {
    if constexpr (LR)
      C.lr.v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                   rlr_b, (lr_lane == 0x80000000u || nb < 0) ? 0x80000000u : lr_lane + uint32_t(nb) * 16u * lr_r * 2,
                   0, 0));
  };

  // Budgets of this block's tokens, published in LDS right before the first row block is
  // multiplied (by then every wave has its first three row blocks in flight): wave 0 clears
  // the table and writes the budget of each token of the block that it holds (in order
  // within the wave, so one barrier suffices).  A token that perm does not name keeps
  // budget 0, so its row is written as zero.  The epilogue reads the table back.
  __shared__ __align__(16) int budT[16 * TB];
  // RT: Wr planes of each wave's tiles and the waves' partial logits
  __shared__ __align__(16) uint16_t wrp[RT ? kMaxWaves : 1][2][3][4][256 + 8];  // rows padded: banks
  __shared__ float lgp[RT ? kMaxWaves : 1][16][4];
  int rbud = 0;  // RT: budget of token (lane & 15), 0 past T
  auto route_budgets = [&]() {
    if constexpr (RT) {
      // every wave holds the same budgets (derived from the same logits) and writes the
      // table it reads itself; no other wave's copy can differ, so no barrier is needed
      if (lane < 16) budT[lane] = rbud;
      return;
    } else if (wave == 0) {
      int pv = pi;
      asm volatile("" : "+v"(pv));  // keep the use of perm (and its wait) here
      int b = 1;
#pragma unroll
      for (int j = 1; j < S; ++j)
        if (off[j] <= lane) b = j + 1;
      const int rr = pv - tb0;
      if (lane < 16 * TB) budT[lane] = 0;
      if (rr >= 0 && rr < Tw) budT[rr] = b;
    }
    __syncthreads();
  };
  const uint32_t lane_code = 16u * lane;
  uint32_t lane_pv[Codes<G, S, TPW, LR>::PH];
#pragma unroll
  for (int h = 0; h < Codes<G, S, TPW, LR>::PH; ++h) {
    const int u = 4 * h + (lane >> 4);
    lane_pv[h] = u < TPW * GPT ? uint32_t(kt[u / GPT] * GPT + u % GPT) * 64u + 4u * (lane & 15) : 0x80000000u;
  }

  // ---- 3. A operands (float32 inputs split into bf16 high and low parts) and the seeds
  // -sum x*o, sum x per group.  Computed inside the streaming loop, after the first weight
  // loads have been issued (see below).
  const u32x4_t bneg0{kNeg128, kNeg32, kNeg8, kNeg128};
  const u32x4_t bneg1{kNeg32, kNeg8, kNeg128, kNeg32};
  const u32x4_t ones{kOnes, kOnes, kOnes, kOnes};
  // Per-group activation sums X[t][g] of the wave's NE groups live in LDS (they are used
  // once per group and row block, by the zero term z * X), token-major so that a lane
  // reads its four tokens with one 16-byte access.
  constexpr int NE = TPW * GPT;
  __shared__ __align__(16) float xsT[kMaxWaves][TB][NE][16];
  f32x4_t gnb[TB][TPW][GPT];
  // The A operands live in the load registers: bf16 activations as loaded, float32 ones
  // (8 values in two registers) split once, in place, into bf16 high and low parts.
  auto aop = [&](int b, int tp, int i, int h, int pa) -> const u32x4_t& { return Araw[b][tp][i][h][pa]; };
  // inputs past K and tiles this wave does not have get zero activations, so their
  // products and sums are exactly zero whatever the redirected loads hold
  auto zero_tile = [&](int b, int tp) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool real = live[tp] && kt[tp] * 256 + xk(i, h) < K;
#pragma unroll
        for (int q = 0; q < NA; ++q)
          if (!real) Araw[b][tp][i][h][q] = u32x4_t{0u, 0u, 0u, 0u};
      }
  };
  auto setup_zero = [&]() {
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int tp = 0; tp < TPW; ++tp) zero_tile(b, tp);
  };
  AF4 af[F4 ? TPW : 1][2];
  // F4: fp8 pairs and scales of one tile's 128-input blocks, then its group sums X on the
  // same instruction with every code 2 (fp4 1.0, B scale 1): X = sum x
  auto f4_tile = [&](int tp) __attribute__((always_inline)) {
    if constexpr (F4) {
      constexpr uint32_t kOne4 = 0x22222222u;
#pragma unroll
      for (int m = 0; m < 2; ++m)
        af[tp][m] = prep_a_f4(Araw[0][tp][2 * m][0][0], Araw[0][tp][2 * m][1][0],
                              Araw[0][tp][2 * m + 1][0][0], Araw[0][tp][2 * m + 1][1][0]);
#pragma unroll
      for (int gi = 0; gi < GPT; ++gi) {
        f32x4_t xs4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          // group gi's inputs within block m: all of it (128, 256) or one half (64)
          if (G == 64 && m != (gi >> 1)) continue;
          if (G == 128 && m != gi) continue;
          const uint32_t lo = (G == 64 && (gi & 1)) ? 0u : kOne4, hi = (G == 64 && !(gi & 1)) ? 0u : kOne4;
          const uint32_t ones[4] = {lo, lo, hi, hi};
          xs4 = mfma_f4<127>(af[tp][m].hi, ones, af[tp][m].sc, xs4);
          xs4 = mfma_f4<127>(af[tp][m].lo, ones, af[tp][m].sc, xs4);
        }
        chain_fence();
        if (r == 0) {
#pragma unroll
          for (int v = 0; v < 4; ++v) xsT[wave][0][tp * GPT + gi][4 * c + v] = xs4[v];
        }
      }
    }
  };
  // bf16 activations are used in place; float32 ones (8 values in two registers) are split
  // once, in place, into bf16 high and low parts
  auto split_x = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (NA == 1) continue;
          const u32x4_t q0 = Araw[b][tp][i][h][0], q1 = Araw[b][tp][i][h][NA - 1];
          u32x4_t hi, lo;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const float v0 = __uint_as_float(d < 2 ? q0[2 * d] : q1[2 * d - 4]);
            const float v1 = __uint_as_float(d < 2 ? q0[2 * d + 1] : q1[2 * d - 3]);
            const uint32_t h0 = bf16_bits_rne(v0), h1 = bf16_bits_rne(v1);
            const uint32_t l0 = bf16_bits_rne(v0 - bf16_bits_to_float(h0));
            const uint32_t l1 = bf16_bits_rne(v1 - bf16_bits_to_float(h1));
            hi[d] = h0 | (h1 << 16);
            lo[d] = l0 | (l1 << 16);
          }
          Araw[b][tp][i][h][0] = hi;
          Araw[b][tp][i][h][NA - 1] = lo;
        }
  };
  auto setup_a = [&]() {
    if constexpr (F4) {
#pragma unroll
      for (int tp = 0; tp < TPW; ++tp) f4_tile(tp);
      return;
    }
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      split_x(b);
#pragma unroll
      for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
        for (int gi = 0; gi < GPT; ++gi) {
          f32x4_t nb4{0.f, 0.f, 0.f, 0.f}, xs4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ii = 0; ii < WPG; ++ii)
#pragma unroll
            for (int pa = 0; pa < NA; ++pa) {
              const int i = gi * WPG + ii;
              nb4 = mfma(aop(b, tp, i, 0, pa), bneg0, nb4);
              nb4 = mfma(aop(b, tp, i, 1, pa), bneg1, nb4);
              xs4 = mfma(aop(b, tp, i, 0, pa), ones, xs4);
              xs4 = mfma(aop(b, tp, i, 1, pa), ones, xs4);
            }
          chain_fence();
          gnb[b][tp][gi] = nb4;
          // lanes (0, c) hold X of tokens 4c + v (every row n sees the same sums)
          if (r == 0) {
#pragma unroll
            for (int v = 0; v < 4; ++v) xsT[wave][b][tp * GPT + gi][4 * c + v] = xs4[v];
          }
        }
    }
    if constexpr (LR) {
      // u as a bf16 hi + lo pair (8 ranks per lane)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float v0 = __uint_as_float(d < 2 ? Uraw[0][2 * d] : Uraw[1][2 * d - 4]);
        const float v1 = __uint_as_float(d < 2 ? Uraw[0][2 * d + 1] : Uraw[1][2 * d - 3]);
        const uint32_t h0 = bf16_bits_rne(v0), h1 = bf16_bits_rne(v1);
        const uint32_t l0 = bf16_bits_rne(v0 - bf16_bits_to_float(h0));
        const uint32_t l1 = bf16_bits_rne(v1 - bf16_bits_to_float(h1));
        Uop[0][d] = h0 | (h1 << 16);
        Uop[1][d] = l0 | (l1 << 16);
      }
    }
  };

  // ---- stream the row blocks.  One buffer resource per slice; a slice no token needs
  // gets an empty range, so its loads return zeros without any memory traffic (and its
  // MFMAs and epilogues are skipped).
  const Magic mg = make_magic();
  __amdgpu_buffer_rsrc_t rs[S];
#pragma unroll
  for (int j = 0; j < S; ++j) rs[j] = slice_rsrc(packed + uint64_t(j) * ss, j < jmax ? uint32_t(ss) : 0u);
  // Three code buffers (two row blocks in flight) unless a wave's registers cannot hold
  // them (group 64 with 4 slices: 32 registers of codes and params per buffer and tile):
  // then two (one row block in flight).
  constexpr bool kThreeBuffers = !(G == 64 && S == 4);
  Codes<G, S, TPW, LR> c0, c1, c2;
  // LR with lr_fz: u is not known while the row blocks stream (Uop stays zero, so the
  // epilogue's side-path MFMAs add nothing and B rows are not loaded).  The storing
  // threads keep each row block's float32 sums in LDS (ystage, row block lr_m of the
  // workgroup) and the side path is added after the last one: see lr_finish_rows.
  int lr_m = 0;
  __shared__ float ystage[LR ? kLrStage : 1][256];
  __shared__ __align__(16) uint32_t ushare[LR ? 64 : 1][8];
  __shared__ u32x4_t bstage[LR ? kLrStage : 1][64];  // wave 0: B rows of staged row block m
  uint32_t* const lr_hdr = reinterpret_cast<uint32_t*>(lr_fz);
  uint64_t* const lr_pairs =
      lrf ? reinterpret_cast<uint64_t*>(lr_fz + kLrPairs) + size_t(blockIdx.y) * 16 * size_t(lr_r) : nullptr;
  // Every workgroup but (0, 0) checks in once it has read E: wave 0, lane 0 sets its own
  // slot to E + 1 (nothing waits for the store).  Workgroup (0, 0), once its u is out,
  // waits until every slot of the launch reads E + 1, then advances E for the next launch:
  // no workgroup reads E after that in this launch, and the next launch starts only after
  // this one ends.
  uint32_t* const lr_slot = reinterpret_cast<uint32_t*>(lr_fz + kLrSlots);
  const uint32_t lr_wg = blockIdx.y * gridDim.x + blockIdx.x, lr_nwg = gridDim.x * gridDim.y;
  auto lr_check_in = [&]() __attribute__((always_inline)) {
    if (wave == 0 && lane == 0 && lr_wg != 0) {
      uint32_t e1 = lrE + 1u;
      asm volatile("" : "+v"(e1));
      __hip_atomic_store(lr_slot + 32 * lr_wg, e1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  auto lr_advance = [&]() __attribute__((always_inline)) {  // wave 0 of workgroup (0, 0)
    if (lr_wg != 0) return;
    const uint32_t want = lrE + 1u;
    for (int it = 0;; ++it) {
      bool ok = true;
      for (uint32_t w = 1 + lane; w < lr_nwg; w += 64)
        ok = ok && __hip_atomic_load(lr_slot + 32 * w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == want;
      if (__ballot(!ok) == 0ull) break;
      if (it >= kLrSpin) {
        if (lane == 0) __hip_atomic_fetch_or(lr_hdr + 2, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
    if (lane == 0) __hip_atomic_store(lr_hdr, want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // Multiplies one row block.  JM, the slices processed, is a compile-time count, so the
  // MFMA chains and epilogues of a group form one straight-line block that the compiler
  // interleaves (a runtime test per slice or tile would split it into small blocks and
  // expose every MFMA's latency).  JM is jmax, the number of slices some token of the
  // batch uses (the loop has one instantiation per value; with the side path only 1 and
  // S, so JM may exceed jmax there); slices past jmax are loaded with
  // an empty buffer range (zeros, no memory traffic) and not multiplied, and a wave
  // without one of its tiles zeroes that tile's scales and zeros.
  auto process = [&](auto jm, const Codes<G, S, TPW, LR>& C, int nb, int buf, Codes<G, S, TPW, LR>& Cn,
                     int nbn) __attribute__((always_inline)) {
    constexpr int JM = decltype(jm)::value;
    // the next buffer's loads (row block nbn) go out first: two row blocks stay in flight
    load_codes(Cn, rs, nbn, kt, KB, NG, uint32_t(po), lane_code, lane_pv);
    load_lr(Cn, nbn);
    f32x4_t acc[TB][JM];
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int j = 0; j < JM; ++j) acc[b][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // this row block's (scale, zero) pairs, unit u of slice j in every lane of row r
    constexpr int PH = Codes<G, S, TPW, LR>::PH;
    uint32_t prm[JM][4 * PH];
#pragma unroll
    for (int j = 0; j < JM; ++j)
#pragma unroll
      for (int h = 0; h < PH; ++h) {
        uint32_t o4[4];
        bcast_rows(C.pw[j][h], o4);
#pragma unroll
        for (int q = 0; q < 4; ++q) prm[j][4 * h + q] = o4[q];
      }
    // One (tile, group) unit at a time: the slices' MFMA chains (one per token block, all
    // fed by the same unpacked codes) are independent and are issued interleaved, then
    // the unit's epilogue scales them into the accumulators.
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int tp = u / GPT, gi = u % GPT;
      f32x4_t P[TB][JM];
#pragma unroll
      for (int b = 0; b < TB; ++b)
#pragma unroll
        for (int j = 0; j < JM; ++j) P[b][j] = F4 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : gnb[b][tp][gi];
      if constexpr (F4) {
        // group gi: 128-input blocks gi (G 128), 0 and 1 (G 256), or one half of block
        // gi >> 1 (G 64: the other half's nibbles zero); every slice's high parts, then
        // every slice's low parts, so the chains interleave
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          if (G == 64 && m != (gi >> 1)) continue;
          if (G == 128 && m != gi) continue;
          uint32_t bw[JM][4];
#pragma unroll
          for (int j = 0; j < JM; ++j) {
            if constexpr (G == 64) {
              const uint32_t w = C.cw[tp][j][gi];
              const bool up = gi & 1;
              bw[j][0] = up ? 0u : f4_even(w);
              bw[j][1] = up ? 0u : f4_odd(w);
              bw[j][2] = up ? f4_even(w) : 0u;
              bw[j][3] = up ? f4_odd(w) : 0u;
            } else {
              const uint32_t w0 = C.cw[tp][j][2 * m], w1 = C.cw[tp][j][2 * m + 1];
              bw[j][0] = f4_even(w0);
              bw[j][1] = f4_odd(w0);
              bw[j][2] = f4_even(w1);
              bw[j][3] = f4_odd(w1);
            }
          }
#pragma unroll
          for (int j = 0; j < JM; ++j) P[0][j] = mfma_f4<128>(af[tp][m].hi, bw[j], af[tp][m].sc, P[0][j]);
#pragma unroll
          for (int j = 0; j < JM; ++j) P[0][j] = mfma_f4<128>(af[tp][m].lo, bw[j], af[tp][m].sc, P[0][j]);
        }
      }
#pragma unroll
      for (int ii = 0; ii < (F4 ? 0 : WPG); ++ii) {
        const int i = gi * WPG + ii;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int j = 0; j < JM; ++j) {
            u32x4_t b0, b1;
            unpack_word(C.cw[tp][j][i], mg, b0, b1);
#pragma unroll
            for (int b = 0; b < TB; ++b)
#pragma unroll
              for (int pa = 0; pa < NA; ++pa) P[b][j] = mfma(aop(b, tp, i, h, pa), h ? b1 : b0, P[b][j]);
          }
        }
      }
      chain_fence();
      // the wave wrote this table itself, so its own in-order LDS accesses suffice
      f32x4_t X4[TB];
#pragma unroll
      for (int b = 0; b < TB; ++b) X4[b] = *reinterpret_cast<const f32x4_t*>(&xsT[wave][b][u][4 * c]);
#pragma unroll
      for (int j = 0; j < JM; ++j) {
        // scale and zero converted once each, then plain fmas (no mixed-precision fma)
        float sc = __half2float(__ushort_as_half(uint16_t(prm[j][u] & 0xFFFFu)));
        float zc = __half2float(__ushort_as_half(uint16_t(prm[j][u] >> 16)));
        asm volatile("" : "+v"(sc), "+v"(zc));
#pragma unroll
        for (int b = 0; b < TB; ++b)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[b][j][v] = fmaf(sc, P[b][j][v], fmaf(zc, X4[b][v], acc[b][j][v]));
      }
    }
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      const int4 bud = *reinterpret_cast<const int4*>(&budT[16 * b + 4 * c]);  // tokens 16b + 4c + v
      f32x4_t out{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < JM; ++j) {
        out[0] += j < bud.x ? acc[b][j][0] : 0.f;
        out[1] += j < bud.y ? acc[b][j][1] : 0.f;
        out[2] += j < bud.z ? acc[b][j][2] : 0.f;
        out[3] += j < bud.w ? acc[b][j][3] : 0.f;
      }
      if constexpr (LR) {
        f32x4_t L = mfma(Uop[0], C.lr.v, f32x4_t{0.f, 0.f, 0.f, 0.f});
        L = mfma(Uop[1], C.lr.v, L);
        chain_fence();
        out[0] += bud.x > 0 ? L[0] : 0.f;
        out[1] += bud.y > 0 ? L[1] : 0.f;
        out[2] += bud.z > 0 ? L[2] : 0.f;
        out[3] += bud.w > 0 ? L[3] : 0.f;
      }
      red[buf][wave][b][lane] = out;
    }
    __syncthreads();
    // one output per thread of the first 4 TB waves (the workgroup has at least that
    // many), so every row block issues a fixed number of stores and the load waits stay
    // exact
    if (threadIdx.x < 256 * TB) {
      const int b = threadIdx.x >> 8, t = threadIdx.x & 255;
      const int p = t >> 4, n16 = t & 15;
      const int ln = 16 * (p >> 2) + n16, v = p & 3;
      float sum = 0.f;
      for (int w = 0; w < NW; ++w) sum += red[buf][w][b][ln][v];
      const int n = nb * 16 + n16, tok = 16 * b + p;
      if (LR && lrf) {
        if (lr_m < kLrStage) {  // finished after the last row block
          ystage[lr_m][threadIdx.x] = sum;
          if constexpr (LR)
            if (wave == 0) bstage[lr_m][lane] = C.lr.v;
        }
      } else if (tok < Tw && n < N) {
        const size_t idx = size_t(tb0 + tok) * N + n;
        if (part)  // one k chunk of several: a float32 partial, summed by splitk_reduce
          part[size_t(blockIdx.z) * T * N + idx] = sum;
        else if (y_bf16)
          reinterpret_cast<uint16_t*>(y)[idx] = uint16_t(bf16_bits_rne(sum));
        else
          reinterpret_cast<float*>(y)[idx] = sum;
      }
    }
    if constexpr (LR) ++lr_m;
  };

  // Three register buffers with fixed roles: step m issues the loads of row block m + 2
  // into buffer (m + 2) % 3 and then multiplies row block m from buffer m % 3, so two row
  // blocks are always in flight.  The prologue loads row blocks 0 and 1, with
  // the seeds and the budgets computed in between (no loads in either).  The loop is
  // instantiated once per slice count read (1 .. S), so
  // inside each copy every path into the loop header carries the same pending loads in
  // the same order, which keeps the compiler's waits on the in-order load counter exact.
  // A load past the end (row block -1) goes out of range: zeros, no memory traffic.
  const int rb0 = lrf ? int(blockIdx.x) - 1 : int(blockIdx.x);
  // (rb0 < 0: the side path's producer, which streams nothing)
  auto nbl = [&](int m) { const int n = rb0 + m * step; return rb0 >= 0 && n < NB ? n : -1; };
  // (scheduling fences keep the issue order perm, x, row block 0, row block 1, so each
  // wait below covers exactly the loads it needs)
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!RT) {
    load_codes(c0, rs, rb0, kt, KB, NG, uint32_t(po), lane_code, lane_pv);
    load_lr(c0, rb0);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (PA) {
    __builtin_amdgcn_sched_barrier(0);
    load_codes(c0, rs, rb0, kt, KB, NG, uint32_t(po), lane_code, lane_pv);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kThreeBuffers) load_codes(c1, rs, nbl(1), kt, KB, NG, uint32_t(po), lane_code, lane_pv);
    __builtin_amdgcn_sched_barrier(0);
    // the prepared operands as they are: A images and scales into the fp8 registers, the
    // group sums into the wave's LDS table, the tiles' partial logits added in tile order
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          af[tp][m].hi[e] = int(pa_x[tp][4 * m][e]);
          af[tp][m].hi[4 + e] = int(pa_x[tp][4 * m + 1][e]);
          af[tp][m].lo[e] = int(pa_x[tp][4 * m + 2][e]);
          af[tp][m].lo[4 + e] = int(pa_x[tp][4 * m + 3][e]);
        }
        af[tp][m].sc = pa_sc[tp][m];
      }
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp)
      if (lane < 16 * GPT) xsT[wave][0][tp * GPT + (lane >> 4)][lane & 15] = __uint_as_float(pa_xs[tp]);
    if (lane < 16) {
      f32x4_t lg4 = __builtin_bit_cast(f32x4_t, pa_lg[0]);
#pragma unroll
      for (int tp = 1; tp < TPW; ++tp) lg4 += __builtin_bit_cast(f32x4_t, pa_lg[tp]);
#pragma unroll
      for (int j = 0; j < S; ++j) lgp[wave][lane][j] = lg4[j];
    }
  } else if constexpr (RT) {
    // Row blocks 0 and 1 go out in here, before the budgets are known, with every slice's
    // range; slices past jmax add nothing there, since no budget reaches them.
    // Wr as three bfloat16 planes (hi + mid + lo = the float32 value: each plane takes the
    // previous one's exact remainder), column-major per tile: wrp[wave][tile][plane][j][k]
    // logits^T = Wr^T x^T on the matrix cores: the activation registers (lane (r, c): token r,
    // 8 inputs per 32-input step) are the B operand as they stand -- setup has already
    // zeroed those of inputs past K and of tiles this wave does not have -- and lane (j, c)
    // of the A operand holds column j of Wr over the same inputs (rows past S repeat a real
    // column; their products land in rows of D nobody reads), so lane (n, 0) ends with
    // token n's S logits.  One accumulator per plane, added lo + mid + hi at the end.
    const int jr = min(r & 3, S - 1);
    f32x4_t Lp[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    // tile by tile, so the first tile's work overlaps the second tile's loads: zero its
    // inputs past K, stage its Wr planes, route it, and (F4) split it into fp8 pairs
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp) {
      zero_tile(0, tp);
#pragma unroll
      for (int q = 0; q < S; ++q)
#pragma unroll
        for (int u = 0; u < 4; u += 2) {
          // floats f, f + 1 of the tile's 256 S (row f / S, column f % S), a pair at a time
          const int f = 4 * (64 * q + lane) + u;
          const float a0 = __uint_as_float(wld[tp][q][u]), b0 = __uint_as_float(wld[tp][q][u + 1]);
          const uint32_t p0 = pk_bf16(a0, b0);
          const float a1 = a0 - __uint_as_float(p0 << 16), b1 = b0 - __uint_as_float(p0 & 0xFFFF0000u);
          const uint32_t p1 = pk_bf16(a1, b1);
          const uint32_t p2 = pk_bf16(a1 - __uint_as_float(p1 << 16), b1 - __uint_as_float(p1 & 0xFFFF0000u));
          wrp[wave][tp][0][f % S][f / S] = uint16_t(p0);
          wrp[wave][tp][1][f % S][f / S] = uint16_t(p1);
          wrp[wave][tp][2][f % S][f / S] = uint16_t(p2);
          wrp[wave][tp][0][(f + 1) % S][(f + 1) / S] = uint16_t(p0 >> 16);
          wrp[wave][tp][1][(f + 1) % S][(f + 1) / S] = uint16_t(p1 >> 16);
          wrp[wave][tp][2][(f + 1) % S][(f + 1) / S] = uint16_t(p2 >> 16);
        }
      // Row blocks 0 and 1 go out once this tile's activations and Wr rows are in (the
      // planes above waited for them), so their HBM round trip runs under the routing
      // MFMAs and the fp8 split; issued earlier, in front of the activation loads of the
      // CU's other waves, they would delay those by a round trip.
      if (tp == 0) {
        __builtin_amdgcn_sched_barrier(0);
        load_codes(c0, rs, rb0, kt, KB, NG, uint32_t(po), lane_code, lane_pv);
        __builtin_amdgcn_sched_barrier(0);
      }
      // Row block 1: every slice now above kLateRow1 tokens; otherwise only its first slice,
      // which every token uses, now and the rest once the budgets are known (below).
      // Either way its slices are pending in slice order when the stream starts.
      if (kThreeBuffers && tp == TPW - 1) {
        __builtin_amdgcn_sched_barrier(0);
        if (T > kLateRow1)
          load_codes(c1, rs, nbl(1), kt, KB, NG, uint32_t(po), lane_code, lane_pv);
        else
          load_codes(c1, rs, nbl(1), kt, KB, NG, uint32_t(po), lane_code, lane_pv, 0, 1);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int kl = xk(i, h);  // first input of the lane's 8 within the tile
#pragma unroll
          for (int pl = 0; pl < 3; ++pl)
            Lp[pl] = mfma(*reinterpret_cast<const u32x4_t*>(&wrp[wave][tp][pl][jr][kl]), Araw[0][tp][i][h][0], Lp[pl]);
        }
      f4_tile(tp);
    }
    chain_fence();
    const f32x4_t L = (Lp[2] + Lp[1]) + Lp[0];
    if (c == 0) {
#pragma unroll
      for (int j = 0; j < S; ++j) lgp[wave][r][j] = L[j];
    }
    if constexpr (!F4) setup_a();
  } else {
    setup_zero();
    setup_a();
  }
  if constexpr (kThreeBuffers && !RT) {
    __builtin_amdgcn_sched_barrier(0);
    load_codes(c1, rs, nbl(1), kt, KB, NG, uint32_t(po), lane_code, lane_pv);
    load_lr(c1, nbl(1));
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (RT) {
    __syncthreads();
    // every lane: token (lane & 15), the waves' partials in wave order
    float lg[S];
#pragma unroll
    for (int j = 0; j < S; ++j) lg[j] = 0.f;
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int j = 0; j < S; ++j) lg[j] += lgp[w][r][j];
    // b = 1 + the first index of the largest logit
    int bb = 1;
    float best = lg[0];
#pragma unroll
    for (int j = 1; j < S; ++j)
      if (lg[j] > best) {
        best = lg[j];
        bb = j + 1;
      }
    rbud = r < T ? bb : 0;
    jmax = 1;
#pragma unroll
    for (int v = 2; v <= S; ++v)
      if (__ballot(lane < T && rbud >= v) != 0ull) jmax = v;
#pragma unroll
    for (int j = 0; j < S; ++j)
      if (j >= jmax) rs[j] = slice_rsrc(packed + uint64_t(j) * ss, 0u);
    if constexpr (!PA && kThreeBuffers) {
      if (T <= kLateRow1) {
        __builtin_amdgcn_sched_barrier(0);
        load_codes(c1, rs, nbl(1), kt, KB, NG, uint32_t(po), lane_code, lane_pv, 1, S);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (blockIdx.x == 0 && blockIdx.z == 0 && wave == 0) {
      // the regroup: stable ascending order by budget, ranks from ballots
      const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
      int base = 0, pos = 0;
      if (lane == 0) rio.offsets[0] = 0;
#pragma unroll
      for (int v = 1; v <= S; ++v) {
        const uint64_t m = __ballot(lane < T && rbud == v);
        if (lane < T && rbud == v) pos = base + __popcll(m & below);
        base += __popcll(m);
        if (lane == 0) rio.offsets[v] = base;
      }
      if (lane < T) {
        rio.perm[pos] = lane;
        rio.budget[lane] = rbud;
#pragma unroll
        for (int j = 0; j < S; ++j) rio.logits[lane * S + j] = lg[j];
      }
    }
  }
  route_budgets();
  auto stream = [&](auto jm) __attribute__((always_inline)) {
    int buf = 0;
    if constexpr (kThreeBuffers) {
      for (int m = 0;; m += 3) {
        process(jm, c0, rb0 + m * step, buf, c2, nbl(m + 2));
        if (rb0 + (m + 1) * step >= NB) break;
        process(jm, c1, rb0 + (m + 1) * step, buf ^ 1, c0, nbl(m + 3));
        if (rb0 + (m + 2) * step >= NB) break;
        process(jm, c2, rb0 + (m + 2) * step, buf, c1, nbl(m + 4));
        buf ^= 1;
        if (rb0 + (m + 3) * step >= NB) break;
      }
    } else {  // two buffers: row block m + 1 loads while m is multiplied
      for (int m = 0;; m += 2) {
        process(jm, c0, rb0 + m * step, 0, c1, nbl(m + 1));
        if (rb0 + (m + 1) * step >= NB) break;
        process(jm, c1, rb0 + (m + 1) * step, 1, c0, nbl(m + 2));
        if (rb0 + (m + 2) * step >= NB) break;
      }
    }
  };
  // one instantiation per slice count read, so the time follows the slices the batch needs
  // (with the side path, whose registers leave no room for more copies, 1 and S only)
  // lr_produce (LR with lr_fz, workgroup 0 of each token block, which streams no row
  // block): u = x A^T of the block's 16 token rows, float32, on the same bf16 MFMA as the
  // codes -- every wave multiplies the activations it holds (prepared as for the stream)
  // by the matching A rows (lane (q, c) of the B operand: rank q, the lane's 8 inputs),
  // the waves' tiles are summed in LDS in wave order, and wave 0 stores u as tagged pairs.
  auto lr_produce = [&]() __attribute__((always_inline)) {
    {
      const __amdgpu_buffer_rsrc_t ra =
          slice_rsrc(reinterpret_cast<const uint8_t*>(lr_a), uint32_t(lr_r) * uint32_t(K) * 2u);
      f32x4_t ua[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        if (16 * f >= lr_r) break;
        const int q = 16 * f + r;
        u32x4_t Af[TPW][4][2];
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int k = kt[tp] * 256 + xk(i, h);
              const uint32_t off =
                  (live[tp] && q < lr_r && k < K) ? (uint32_t(q) * uint32_t(K) + uint32_t(k)) * 2u : 0x80000000u;
              Af[tp][i][h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0));
            }
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int pa = 0; pa < NA; ++pa) ua[f] = mfma(aop(0, tp, i, h, pa), Af[tp][i][h], ua[f]);
      }
      chain_fence();
      red[0][wave][0][lane] = ua[0];
      red[1][wave][0][lane] = ua[1];
      __syncthreads();
      if (wave == 0) {
        const uint64_t tag = uint64_t(lrE + 1u) << 32;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int q = 16 * f + r;
          if (16 * f < lr_r) {
            f32x4_t sm = red[f][0][0][lane];
            for (int w = 1; w < NW; ++w) sm += red[f][w][0][lane];
            if (q < lr_r) {
#pragma unroll
              for (int v = 0; v < 4; ++v)  // lane (q, c) holds tokens 4c + v
                __hip_atomic_store(lr_pairs + (4 * c + v) * lr_r + q, tag | uint64_t(__float_as_uint(sm[v])),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
        lr_advance();
      }
    }
  };

  auto run = [&]() __attribute__((always_inline)) {
    if constexpr (S >= 2)
      if (jmax == 1) return stream(std::integral_constant<int, 1>{});
    if constexpr (S >= 3 && !LR)
      if (jmax == 2) return stream(std::integral_constant<int, 2>{});
    if constexpr (S >= 4 && !LR)
      if (jmax == 3) return stream(std::integral_constant<int, 3>{});
    stream(std::integral_constant<int, S>{});
  };
  if (lrf && blockIdx.x == 0) {
    if constexpr (LR) {
      lr_check_in();
      lr_produce();
    }
    return;
  }
  if constexpr (LR)
    if (lrf) lr_check_in();
  run();
  // lr_finish_rows (LR with lr_fz): wave 0 waits (bounded) for this launch's u, turns it
  // into the MFMA's bf16 hi + lo pairs and shares them through LDS; each wave then adds
  // u . B^T of row blocks m = wave, wave + NW, ... to the staged sums (tokens whose budget
  // is 0 are left out, as in the epilogue), and the storing threads write every row
  // block once, rounded once.  If u never comes, the side path is left out and error
  // bit 0 is set rather than waiting forever.
  if constexpr (LR) {
    if (lrf) {
      const int nst = min(lr_m, kLrStage);
      if (wave == 0) {
        const uint32_t want = lrE + 1u;
        uint64_t pv[8];
        for (int it = 0;; ++it) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pv[e] = 8 * c < lr_r ? __hip_atomic_load(lr_pairs + r * lr_r + 8 * c + e, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT)
                                 : 0;
          bool ok = true;
#pragma unroll
          for (int e = 0; e < 8; ++e) ok = ok && (8 * c >= lr_r || uint32_t(pv[e] >> 32) == want);
          if (__ballot(!ok) == 0ull) break;
          if (it >= kLrSpin) {
            if (lane == 0) __hip_atomic_fetch_or(lr_hdr + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int e = 0; e < 8; ++e) pv[e] = 0;
            break;
          }
          __builtin_amdgcn_s_sleep(8);
        }
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float v0 = __uint_as_float(uint32_t(pv[2 * d])), v1 = __uint_as_float(uint32_t(pv[2 * d + 1]));
          const uint32_t h0 = bf16_bits_rne(v0), h1 = bf16_bits_rne(v1);
          const uint32_t l0 = bf16_bits_rne(v0 - bf16_bits_to_float(h0));
          const uint32_t l1 = bf16_bits_rne(v1 - bf16_bits_to_float(h1));
          ushare[lane][d] = h0 | (h1 << 16);
          ushare[lane][4 + d] = l0 | (l1 << 16);
        }
      }
      __syncthreads();
      const u32x4_t uh = *reinterpret_cast<const u32x4_t*>(&ushare[lane][0]);
      const u32x4_t ul = *reinterpret_cast<const u32x4_t*>(&ushare[lane][4]);
      auto add_lr = [&](int m, const u32x4_t& bm) __attribute__((always_inline)) {
        f32x4_t L = mfma(uh, bm, f32x4_t{0.f, 0.f, 0.f, 0.f});
        L = mfma(ul, bm, L);
        chain_fence();
#pragma unroll
        for (int v = 0; v < 4; ++v)  // lane (n, c): tokens 4c + v of output row n
          if (budT[4 * c + v] > 0) ystage[m][(4 * c + v) * 16 + r] += L[v];
      };
      for (int m = wave; m < nst; m += NW) add_lr(m, bstage[m][lane]);
      __syncthreads();
      if (threadIdx.x < 256) {
        const int p = threadIdx.x >> 4, n16 = threadIdx.x & 15;
        if (p < Tw)
          for (int m = 0; m < nst; ++m) {
            const int n = (rb0 + m * step) * 16 + n16;
            if (n < N) {
              const size_t idx = size_t(tb0 + p) * N + n;
              const float val = ystage[m][threadIdx.x];
              if (y_bf16)
                reinterpret_cast<uint16_t*>(y)[idx] = uint16_t(bf16_bits_rne(val));
              else
                reinterpret_cast<float*>(y)[idx] = val;
            }
          }
      }
    }
  }
}

// Whether the preparing launch gives each 128-input block of a k tile its own fp8 wave
// (two or more groups per tile, so no group spans both blocks).
constexpr bool prep_split(int G) { return G <= 128; }

// The first launch of the two-launch decode step (PA): a workgroup per k tile of 256 inputs
// prepares what every workgroup of the streaming kernel would otherwise derive from the
// raw activations on its own.  Waves 1 and 2 take the fp8 A operands (prep_a_f4) of the
// tile's two 128-input blocks and their group sums (the same instruction against all-ones
// codes; wave 1 takes both blocks with groups of 256); wave 0, in parallel, the
// tile's partial router logits (Wr as three exact bfloat16 planes on the bf16 matrix
// instruction, as in the in-kernel routing).  bfloat16 x [t x K], t <= 16; tokens past t
// repeat the last one (their rows are never used).  Output layout: PrepLayout.
template <int G, int S>
__global__ __launch_bounds__(192) void decode_prep_kernel(const uint8_t* __restrict__ x, int T, int K, int KB,
                                                          const float* __restrict__ wr, uint8_t* __restrict__ prep) {
  asm volatile("" ::"s"(x), "s"(wr), "s"(prep), "s"(T), "s"(K), "s"(KB));
  constexpr int GPT = 256 / G;
  const int t = blockIdx.x, lane = threadIdx.x & 63, r = lane & 15, c = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int xr = min(r, T - 1);
  auto xk = [&](int i, int h) { return 128 * (i >> 1) + 64 * (c & 1) + 16 * (c >> 1) + 32 * (i & 1) + 8 * h; };
  u32x4_t a[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = t * 256 + xk(i, h);
      a[i][h] = ldg16(x + (size_t(xr) * K + (k < K ? k : 0)) * 2);   // past K: zeroed below
    }
  const PrepLayout pl(KB, G);
  if (wv == 0) {
    const __amdgpu_buffer_rsrc_t rw = slice_rsrc(reinterpret_cast<const uint8_t*>(wr), uint32_t(K) * S * 4);
    u32x4_t wl[S];
#pragma unroll
    for (int q = 0; q < S; ++q)
      wl[q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, (uint32_t(t) * 256 * S + (64 * q + lane) * 4) * 4, 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (t * 256 + xk(i, h) >= K) a[i][h] = u32x4_t{0u, 0u, 0u, 0u};
    // Wr rows of the tile as three bf16 planes, column-major (plane, logit, input), in LDS;
    // logits^T = Wr^T x^T with the activations as the B operand (see the in-kernel routing)
    __shared__ __align__(16) uint16_t wrp[3][4][256 + 8];
#pragma unroll
    for (int q = 0; q < S; ++q)
#pragma unroll
      for (int u = 0; u < 4; u += 2) {
        const int f = 4 * (64 * q + lane) + u;
        const float a0 = __uint_as_float(wl[q][u]), b0 = __uint_as_float(wl[q][u + 1]);
        const uint32_t p0 = pk_bf16(a0, b0);
        const float a1 = a0 - __uint_as_float(p0 << 16), b1 = b0 - __uint_as_float(p0 & 0xFFFF0000u);
        const uint32_t p1 = pk_bf16(a1, b1);
        const uint32_t p2 = pk_bf16(a1 - __uint_as_float(p1 << 16), b1 - __uint_as_float(p1 & 0xFFFF0000u));
        wrp[0][f % S][f / S] = uint16_t(p0);
        wrp[1][f % S][f / S] = uint16_t(p1);
        wrp[2][f % S][f / S] = uint16_t(p2);
        wrp[0][(f + 1) % S][(f + 1) / S] = uint16_t(p0 >> 16);
        wrp[1][(f + 1) % S][(f + 1) / S] = uint16_t(p1 >> 16);
        wrp[2][(f + 1) % S][(f + 1) / S] = uint16_t(p2 >> 16);
      }
    const int jr = min(r & 3, S - 1);
    f32x4_t Lp[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int pn = 0; pn < 3; ++pn)
          Lp[pn] = mfma(*reinterpret_cast<const u32x4_t*>(&wrp[pn][jr][xk(i, h)]), a[i][h], Lp[pn]);
    chain_fence();
    const f32x4_t L = (Lp[2] + Lp[1]) + Lp[0];
    // lanes (n, 0) hold token n's logits
    if (c == 0) reinterpret_cast<f32x4_t*>(prep + pl.lg)[size_t(t) * 16 + r] = L;
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (t * 256 + xk(i, h) >= K) a[i][h] = u32x4_t{0u, 0u, 0u, 0u};
  // fp8 pairs and scales of the 128-input blocks, then their group sums.  With two or more
  // groups per tile the blocks are independent: wave 1 + m takes block m (prep_split);
  // with one group of 256 wave 1 takes both.
  const int m_lo = prep_split(G) ? wv - 1 : 0, m_hi = prep_split(G) ? wv : 2;
  AF4 af[2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
    if (m >= m_lo && m < m_hi) af[m] = prep_a_f4(a[2 * m][0], a[2 * m][1], a[2 * m + 1][0], a[2 * m + 1][1]);
  constexpr uint32_t kOne4 = 0x22222222u;
  f32x4_t xs[GPT];
#pragma unroll
  for (int gi = 0; gi < GPT; ++gi) {
    xs[gi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (m < m_lo || m >= m_hi) continue;
      if (G == 64 && m != (gi >> 1)) continue;
      if (G == 128 && m != gi) continue;
      const uint32_t lo = (G == 64 && (gi & 1)) ? 0u : kOne4, hi = (G == 64 && !(gi & 1)) ? 0u : kOne4;
      const uint32_t ones[4] = {lo, lo, hi, hi};
      xs[gi] = mfma_f4<127>(af[m].hi, ones, af[m].sc, xs[gi]);
      xs[gi] = mfma_f4<127>(af[m].lo, ones, af[m].sc, xs[gi]);
    }
  }
  chain_fence();
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    if (m < m_lo || m >= m_hi) continue;
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(prep + pl.a) + (size_t(t) * 8 + 4 * m) * 64 + lane;
    dst[0] = u32x4_t{uint32_t(af[m].hi[0]), uint32_t(af[m].hi[1]), uint32_t(af[m].hi[2]), uint32_t(af[m].hi[3])};
    dst[64] = u32x4_t{uint32_t(af[m].hi[4]), uint32_t(af[m].hi[5]), uint32_t(af[m].hi[6]), uint32_t(af[m].hi[7])};
    dst[128] = u32x4_t{uint32_t(af[m].lo[0]), uint32_t(af[m].lo[1]), uint32_t(af[m].lo[2]), uint32_t(af[m].lo[3])};
    dst[192] = u32x4_t{uint32_t(af[m].lo[4]), uint32_t(af[m].lo[5]), uint32_t(af[m].lo[6]), uint32_t(af[m].lo[7])};
  }
#pragma unroll
  for (int m = 0; m < 2; ++m)
    if (m >= m_lo && m < m_hi) reinterpret_cast<uint32_t*>(prep + pl.sc)[(size_t(t) * 64 + lane) * 2 + m] = af[m].sc;
  // lanes (0, c) hold the group sums of tokens 4c .. 4c + 3 (of the wave's groups)
  if (r == 0) {
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      const int m = G == 64 ? gi >> 1 : (G == 128 ? gi : 0);
      if (prep_split(G) && (m < m_lo || m >= m_hi)) continue;
      *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(prep + pl.xs) + (size_t(t) * GPT + gi) * 16 + 4 * c) = xs[gi];
    }
  }
}

// Sums the k chunks' float32 partials in a fixed order (deterministic) and writes y.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int ks,
                                                            size_t tn, void* __restrict__ y,
                                                            int y_bf16) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < tn; i += size_t(gridDim.x) * 256) {
    float sum = part[i];
    for (int z = 1; z < ks; ++z) sum += part[size_t(z) * tn + i];
    if (y_bf16)
      reinterpret_cast<uint16_t*>(y)[i] = uint16_t(bf16_bits_rne(sum));
    else
      reinterpret_cast<float*>(y)[i] = sum;
  }
}

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

// Whether a wave can hold two k tiles (their activations, seeds and three buffers of codes
// and params) in its 256 registers without spilling.  A spill would wait on the in-order
// load counter behind the prefetched weights; the build checks that every instantiated
// variant is spill-free.
constexpr bool two_tiles_fit(int G, int S, int NA) {
  return NA == 1 ? (G == 64 ? S <= 1 : S <= 3) : (G == 128 ? S <= 1 : (G == 256 && S <= 2));
}

// Whether a wave can hold two 16-token blocks (one k tile): bf16 activations with one
// slice at group 64, up to three at group 128 and up to four at group 256.
constexpr bool two_blocks_fit(int G, int S, int NA) {
  return NA == 1 && (G == 64 ? S == 1 : (G == 128 ? S <= 3 : S <= 4));
}

// Group 64 with 4 slices and float32 activations does not fit a wave's registers even
// with two buffers; the generic decode kernel serves it.
constexpr bool stream_fits(int G, int S, int NA) { return !(G == 64 && S == 4 && NA == 2); }

// Variants that carry the side path: every streaming variant with one token block per
// workgroup, and two k tiles per wave where its 20 more registers still fit (group 256
// with 2 slices and float32 activations would spill).
constexpr bool lr_fits(int G, int S, int NA) { return stream_fits(G, S, NA); }
constexpr bool lr_two_tiles_fit(int G, int S, int NA) {
  return two_tiles_fit(G, S, NA) && !(G == 256 && S == 2 && NA == 2);
}

// How a launch covers the tokens and k tiles.  Batches of more than 32 tokens put two
// 16-token blocks in each workgroup (TB = 2) where the registers allow, so the codes are
// unpacked (and read from L2) once for both; a wave then holds one k tile, so K may need
// more chunks.  Up to 32 tokens the extra chunks would cost more than the shared unpack
// saves when few slices are read, so those batches keep one block per workgroup.  One workgroup holds up to 8
// waves x TPW tiles; a longer K is cut into ks equal chunks (grid z) whose float32
// partials go to the workspace.
struct Plan {
  int tb, tpw, kchunk, ks, nw;
};

// With the side path (lr) every variant takes one token block per workgroup.
Plan make_plan(const mbq_desc& d, int32_t t, bool x_bf16, bool lr) {
  const int na = x_bf16 ? 1 : 2;
  const int tb = (!lr && t > 32 && two_blocks_fit(d.group, d.slices, na)) ? 2 : 1;
  const bool two = lr ? lr_two_tiles_fit(d.group, d.slices, na) : two_tiles_fit(d.group, d.slices, na);
  const int tmax = (tb == 1 && two) ? 2 : 1;
  const int kb = d.k_tiles;
  int ks = (kb + kMaxWaves * tmax - 1) / (kMaxWaves * tmax);
  const int kchunk = (kb + ks - 1) / ks;
  ks = (kb + kchunk - 1) / kchunk;
  const int tpw = kchunk > kMaxWaves ? 2 : 1;
  const int nw = std::max(4 * tb, (kchunk + tpw - 1) / tpw);  // >= 4 TB waves: the store step
  return Plan{tb, tpw, kchunk, ks, nw};
}


struct LrArgs {
  const float* u;
  int ks;
  const uint16_t* b;
  int r;
  uint8_t* fz;         // non-null: u computed inside the launch (see lr_produce), state here
  const uint16_t* a;   // A [r x K], with fz
};

template <int G, int S, int NA, int TPW, int TB, bool LR, bool RT = false, bool F4 = false, bool PA = false>
hipError_t launch_gsn(const mbq_desc& d, const Plan& pl, const void* packed, int32_t t,
                      const void* x, const int32_t* perm, const int32_t* offsets, void* y,
                      bool y_bf16, float* part, const LrArgs& lr, hipStream_t stream,
                      const RouteIO& rio = RouteIO{}) {
  // One workgroup per CU.  The token-block groups and k chunks of a launch share the CUs,
  // so they all run at once: with gridDim.x a multiple of 8, workgroups (x, y, z) of every
  // y and z sit on XCD x % 8, and the token groups of one k chunk walk the same row blocks
  // at the same pace, so each weight line comes from HBM once and is served to the other
  // token groups by that XCD's L2.
  const int ty = (t + 16 * TB - 1) / (16 * TB);
  const int cap = std::max(8, (cu_count() / (ty * pl.ks)) & ~7);
  // with u computed inside the launch, workgroup 0 of each token block computes it and
  // the others stream: one CU of the cap goes to it
  const bool fz = LR && lr_inline_fits(NA, TPW) && lr.fz != nullptr;
  const int grid = fz ? std::min(d.row_blocks, cap - 1) + 1 : std::min(d.row_blocks, cap);
  hipLaunchKernelGGL((decode_stream_kernel<G, S, NA, TPW, TB, LR, RT, F4, PA>), dim3(grid, ty, pl.ks), dim3(64 * pl.nw),
                     0, stream, static_cast<const uint8_t*>(packed), d.n, d.k, d.k_tiles,
                     d.groups_padded, d.row_blocks, d.slice_stride, d.params_offset, x, t, perm,
                     offsets, y, int(y_bf16), pl.kchunk, part, lr.u, lr.ks, lr.b, lr.r,
                     fz ? lr.fz : nullptr, lr.a, rio);
  return hipGetLastError();
}

template <int G, int S, int NA>
hipError_t launch_gs(const mbq_desc& d, const Plan& pl, const void* packed, int32_t t,
                     const void* x, const int32_t* perm, const int32_t* offsets, void* y,
                     bool y_bf16, float* part, const LrArgs& lr, hipStream_t stream) {
  if constexpr (lr_fits(G, S, NA)) {
    if (lr.r > 0) {
      if constexpr (lr_two_tiles_fit(G, S, NA)) {
        if (pl.tpw == 2)
          return launch_gsn<G, S, NA, 2, 1, true>(d, pl, packed, t, x, perm, offsets, y, y_bf16, part, lr, stream);
      }
      return launch_gsn<G, S, NA, 1, 1, true>(d, pl, packed, t, x, perm, offsets, y, y_bf16, part, lr, stream);
    }
  }
  if constexpr (two_blocks_fit(G, S, NA)) {
    if (pl.tb == 2)
      return launch_gsn<G, S, NA, 1, 2, false>(d, pl, packed, t, x, perm, offsets, y, y_bf16, part, lr, stream);
  }
  if constexpr (two_tiles_fit(G, S, NA)) {
    if (pl.tpw == 2)
      return launch_gsn<G, S, NA, 2, 1, false>(d, pl, packed, t, x, perm, offsets, y, y_bf16, part, lr, stream);
  }
  return launch_gsn<G, S, NA, 1, 1, false>(d, pl, packed, t, x, perm, offsets, y, y_bf16, part, lr, stream);
}


// In-kernel routing: bfloat16 activations, one token block, no side path, one k chunk.
// f4 selects the fp8 x fp4 multiply (see above); pa (with f4) the two-launch step:
// decode_prep_kernel, then the streaming kernel on its prepared operands.
template <int G, int S>
hipError_t launch_route_gs(const mbq_desc& d, const Plan& pl, const void* packed, int32_t t,
                           const void* x, void* y, bool y_bf16, const RouteIO& rio, bool f4, bool pa,
                           hipStream_t stream) {
  if constexpr (stream_fits(G, S, 1)) {
    if constexpr (two_tiles_fit(G, S, 1)) {
      if (pl.tpw == 2) {
        if (f4 && pa)
          return launch_gsn<G, S, 1, 2, 1, false, true, true, true>(d, pl, packed, t, x, nullptr, nullptr, y,
                                                                    y_bf16, nullptr, LrArgs{}, stream, rio);
        if (f4)
          return launch_gsn<G, S, 1, 2, 1, false, true, true>(d, pl, packed, t, x, nullptr, nullptr, y, y_bf16,
                                                              nullptr, LrArgs{}, stream, rio);
        return launch_gsn<G, S, 1, 2, 1, false, true>(d, pl, packed, t, x, nullptr, nullptr, y, y_bf16,
                                                      nullptr, LrArgs{}, stream, rio);
      }
    }
    if (f4 && pa)
      return launch_gsn<G, S, 1, 1, 1, false, true, true, true>(d, pl, packed, t, x, nullptr, nullptr, y, y_bf16,
                                                                nullptr, LrArgs{}, stream, rio);
    if (f4)
      return launch_gsn<G, S, 1, 1, 1, false, true, true>(d, pl, packed, t, x, nullptr, nullptr, y, y_bf16,
                                                          nullptr, LrArgs{}, stream, rio);
    return launch_gsn<G, S, 1, 1, 1, false, true>(d, pl, packed, t, x, nullptr, nullptr, y, y_bf16,
                                                  nullptr, LrArgs{}, stream, rio);
  }
  return hipErrorInvalidValue;  // excluded by decode_route_supported
}

template <int G>
hipError_t launch_prep_g(const mbq_desc& d, int32_t t, const void* x, const float* wr, void* prep,
                         hipStream_t stream) {
  const auto x8 = static_cast<const uint8_t*>(x);
  auto p8 = static_cast<uint8_t*>(prep);
  // per k tile: a routing wave and one fp8 wave per 128-input block (one for both at group 256)
  const dim3 grid(d.k_tiles), block(prep_split(G) ? 192 : 128);
  switch (d.slices) {
    case 2: hipLaunchKernelGGL((decode_prep_kernel<G, 2>), grid, block, 0, stream, x8, t, d.k, d.k_tiles, wr, p8); break;
    case 3: hipLaunchKernelGGL((decode_prep_kernel<G, 3>), grid, block, 0, stream, x8, t, d.k, d.k_tiles, wr, p8); break;
    default: hipLaunchKernelGGL((decode_prep_kernel<G, 4>), grid, block, 0, stream, x8, t, d.k, d.k_tiles, wr, p8); break;
  }
  return hipGetLastError();
}

template <int G>
hipError_t launch_route_g(const mbq_desc& d, const Plan& pl, const void* packed, int32_t t,
                          const void* x, void* y, bool y_bf16, const RouteIO& rio, bool f4, bool pa,
                          hipStream_t stream) {
  switch (d.slices) {
    case 1: return launch_route_gs<G, 1>(d, pl, packed, t, x, y, y_bf16, rio, false, false, stream);
    case 2: return launch_route_gs<G, 2>(d, pl, packed, t, x, y, y_bf16, rio, f4, pa, stream);
    case 3: return launch_route_gs<G, 3>(d, pl, packed, t, x, y, y_bf16, rio, f4, pa, stream);
    default: return launch_route_gs<G, 4>(d, pl, packed, t, x, y, y_bf16, rio, f4, pa, stream);
  }
}

template <int G, int NA>
hipError_t launch_gn(const mbq_desc& d, const Plan& pl, const void* packed, int32_t t,
                     const void* x, const int32_t* perm, const int32_t* offsets, void* y,
                     bool y_bf16, float* part, const LrArgs& lr, hipStream_t stream) {
  switch (d.slices) {
    case 1: return launch_gs<G, 1, NA>(d, pl, packed, t, x, perm, offsets, y, y_bf16, part, lr, stream);
    case 2: return launch_gs<G, 2, NA>(d, pl, packed, t, x, perm, offsets, y, y_bf16, part, lr, stream);
    case 3: return launch_gs<G, 3, NA>(d, pl, packed, t, x, perm, offsets, y, y_bf16, part, lr, stream);
    default:
      if constexpr (stream_fits(G, 4, NA))
        return launch_gs<G, 4, NA>(d, pl, packed, t, x, perm, offsets, y, y_bf16, part, lr, stream);
      return hipErrorInvalidValue;  // excluded by decode_stream_supported
  }
}

template <int G>
hipError_t launch_g(const mbq_desc& d, const Plan& pl, const void* packed, int32_t t,
                    const void* x, bool x_bf16, const int32_t* perm, const int32_t* offsets,
                    void* y, bool y_bf16, float* part, const LrArgs& lr, hipStream_t stream) {
  if (x_bf16) return launch_gn<G, 1>(d, pl, packed, t, x, perm, offsets, y, y_bf16, part, lr, stream);
  return launch_gn<G, 2>(d, pl, packed, t, x, perm, offsets, y, y_bf16, part, lr, stream);
}

}  // namespace

bool decode_stream_supported(const mbq_desc& d, int32_t t, bool x_bf16, bool lr) {
  // buffer offsets are 32-bit: a slice must stay below 4 GiB
  const int na = x_bf16 ? 1 : 2;
  // groups of 32 inputs split a lane's code word in two: served by the generic kernel
  return t >= 1 && t <= kMaxTokens && d.group >= 64 && d.slice_stride < (uint64_t(1) << 32) &&
         (lr ? lr_fits(d.group, d.slices, na) : stream_fits(d.group, d.slices, na));
}

bool decode_route_supported(const mbq_desc& d, int32_t t) {
  if (t < 1 || t > 16 || !decode_stream_supported(d, t, true, false)) return false;
  const Plan pl = make_plan(d, t, true, false);
  return pl.ks == 1 && pl.tb == 1;
}

size_t decode_route_workspace(const mbq_desc& d, int32_t t) {
  return decode_prepared_supported(d, t) ? PrepLayout(d.k_tiles, d.group).bytes : 0;
}

bool decode_prepared_supported(const mbq_desc& d, int32_t t) {
  return d.slices >= 2 && decode_route_supported(d, t);
}

hipError_t launch_decode_prepare(const mbq_desc& d, int32_t t, const void* x, const float* wr, void* prep,
                                 hipStream_t stream) {
  switch (d.group) {
    case 64: return launch_prep_g<64>(d, t, x, wr, prep, stream);
    case 128: return launch_prep_g<128>(d, t, x, wr, prep, stream);
    default: return launch_prep_g<256>(d, t, x, wr, prep, stream);
  }
}

hipError_t launch_decode_prepared(const mbq_desc& d, const void* packed, int32_t t, const void* prep,
                                  float* logits, int32_t* budget, int32_t* perm, int32_t* offsets, void* y,
                                  bool y_bf16, hipStream_t stream) {
  const RouteIO rio{nullptr, logits, budget, perm, offsets, static_cast<const uint8_t*>(prep)};
  const Plan pl = make_plan(d, t, true, false);
  switch (d.group) {
    case 64: return launch_route_g<64>(d, pl, packed, t, nullptr, y, y_bf16, rio, true, true, stream);
    case 128: return launch_route_g<128>(d, pl, packed, t, nullptr, y, y_bf16, rio, true, true, stream);
    default: return launch_route_g<256>(d, pl, packed, t, nullptr, y, y_bf16, rio, true, true, stream);
  }
}

hipError_t launch_decode_route(const mbq_desc& d, const void* packed, int32_t t, const void* x,
                               const float* wr, float* logits, int32_t* budget, int32_t* perm,
                               int32_t* offsets, void* y, bool y_bf16, int mul, int launches, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  // Two launches (decode_prep_kernel prepares the fp8 operands, the partial logits and the
  // group sums once, instead of in every workgroup) pay from about 10 tokens: below, the
  // second launch costs more than the per-workgroup preparation it saves (18944 x 3584,
  // graph replays, one launch against two: 19.6 / 20.3 us at 5 tokens, 20.2 / 20.4 at 8,
  // 20.9 / 20.7 at 12, 21.6 / 20.5 at 16).
  const bool room = ws && ws_bytes >= PrepLayout(d.k_tiles, d.group).bytes;
  bool pa = launches == 2 || (launches == 0 && t > 8 && room);
  const RouteIO rio{wr, logits, budget, perm, offsets, static_cast<const uint8_t*>(ws)};
  const Plan pl = make_plan(d, t, true, false);
  // The fp8 x fp4 multiply saves ~1/4 of a row block's time but its activation split
  // costs every workgroup about two row blocks' worth up front: taken from 4 row blocks
  // per workgroup, 2 slices and 2 tokens on (one token reads one slice more often than
  // not; on the 18944 x 3584 weight, bf16 against fp8 x fp4 in one launch: 13.7 / 14.1 us
  // at 1 token, 16.6 / 15.7 at 2, 16.4 / 15.7 at 3, 20.2 / 19.5 at 4), unless the
  // caller chooses (mul).
  const int grid = std::min(d.row_blocks, std::max(8, cu_count() & ~7));
  bool f4 = d.slices >= 2 && t >= 2 && (d.row_blocks + grid - 1) / grid >= 4;
  if (mul == MBQ_MUL_BF16) f4 = false;
  if (mul == MBQ_MUL_FP8_FP4) f4 = true;
  if (!f4 || d.slices < 2) pa = false;
  if (pa) {
    const hipError_t e = launch_decode_prepare(d, t, x, wr, ws, stream);
    if (e != hipSuccess) return e;
    return launch_decode_prepared(d, packed, t, ws, logits, budget, perm, offsets, y, y_bf16, stream);
  }
  switch (d.group) {
    case 64: return launch_route_g<64>(d, pl, packed, t, x, y, y_bf16, rio, f4, pa, stream);
    case 128: return launch_route_g<128>(d, pl, packed, t, x, y, y_bf16, rio, f4, pa, stream);
    default: return launch_route_g<256>(d, pl, packed, t, x, y, y_bf16, rio, f4, pa, stream);
  }
}

size_t decode_stream_workspace(const mbq_desc& d, int32_t t, bool x_bf16, bool lr) {
  const Plan pl = make_plan(d, t, x_bf16, lr);
  return pl.ks > 1 ? size_t(pl.ks) * size_t(t) * size_t(d.n) * sizeof(float) : 0;
}

// The side path's u computed inside the streaming launch needs all of K in one
// workgroup (every token block's workgroup 0 multiplies the whole row of activations)
// and every streaming workgroup's row blocks held in LDS until u is added.
bool decode_stream_lr_inline(const mbq_desc& d, int32_t t, bool x_bf16) {
  if (!decode_stream_supported(d, t, x_bf16, true)) return false;
  const Plan pl = make_plan(d, t, x_bf16, true);
  if (pl.ks != 1 || !lr_inline_fits(x_bf16 ? 1 : 2, pl.tpw)) return false;
  const int ty = (t + 15) / 16;
  const int cap = std::max(8, (cu_count() / ty) & ~7);
  const int streaming = std::min(d.row_blocks, cap - 1);  // as in launch_gsn
  return streaming >= 1 && (d.row_blocks + streaming - 1) / streaming <= kLrStage &&
         (streaming + 1) * ty <= kLrMaxWg;
}

hipError_t launch_decode_stream(const mbq_desc& d, const void* packed, int32_t t, const void* x,
                                bool x_bf16, const int32_t* perm, const int32_t* offsets,
                                void* y, bool y_bf16, void* workspace, const float* lr_u,
                                int32_t lr_ks, const uint16_t* lr_b, int32_t lr_r, uint8_t* lr_fz,
                                const uint16_t* lr_a, hipStream_t stream) {
  const LrArgs lr{lr_u, lr_ks, lr_b, lr_r, lr_fz, lr_a};
  const Plan pl = make_plan(d, t, x_bf16, lr_r > 0);
  float* part = pl.ks > 1 ? static_cast<float*>(workspace) : nullptr;
  hipError_t e;
  switch (d.group) {
    case 64: e = launch_g<64>(d, pl, packed, t, x, x_bf16, perm, offsets, y, y_bf16, part, lr, stream); break;
    case 128: e = launch_g<128>(d, pl, packed, t, x, x_bf16, perm, offsets, y, y_bf16, part, lr, stream); break;
    default: e = launch_g<256>(d, pl, packed, t, x, x_bf16, perm, offsets, y, y_bf16, part, lr, stream); break;
  }
  if (e != hipSuccess || !part) return e;
  const size_t tn = size_t(t) * size_t(d.n);
  const int blocks = int(std::min<size_t>((tn + 255) / 256, size_t(8) * cu_count()));
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, stream, part, pl.ks, tn, y,
                     int(y_bf16));
  return hipGetLastError();
}

}  // namespace mbq
