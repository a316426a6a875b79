// Routed decode linear for small batches (T <= 16) -- the HBM-streaming kernel.
//
// Same arithmetic as decode.hip (MoBiQuant explainer, gist.science English page, sections
// 2.A and 3: each token sums its own slices; only slices some token uses are fetched):
//   y[t, n] = sum_j [b(t) >= j] sum_g ( s_jng * P_jng[t] + z_jng * X_g[t] ),
//   P = sum_{k in g} x_k q_k on MFMA 16x16x32 bf16 with raw codes as bf16 (o + q) values
//   and the accumulator seeded with -sum_k x_k o_k.
//
// Organisation (one persistent workgroup per CU):
//   * wave w owns k tiles w, w + NW, ... (TPW of them): their slice of x (the A operand)
//     and the per-group seeds -sum x*o and sum x are computed once and stay in registers
//     for the whole kernel.  With at most 16 tokens there is a single MFMA token block, so
//     rows stay in the tokens' original order: x is read with no dependence on perm, and
//     perm / offsets only decide which slices count for which row;
//   * the workgroup walks row blocks nb = blockIdx.x, + gridDim.x, ...; for each, every
//     wave multiplies its k tiles of every needed slice while the next two row blocks'
//     codes and params are already loading (three register buffers with fixed roles,
//     every load unconditional: an unused slice or a past-the-end row block re-reads
//     cached lines);
//   * the waves' partial 16x16 tiles are summed in LDS (double-buffered, one barrier per
//     row block) and written out with per-token slice masks already applied.
// Token perm[i] (sorted position i) has budget b with offsets[b-1] <= i < offsets[b].
#include "mbq_internal.h"

namespace mbq {
namespace {

constexpr int kMaxWaves = 8;
constexpr uint32_t kNeg128 = 0xC300C300u, kNeg32 = 0xC200C200u, kNeg8 = 0xC100C100u;
constexpr uint32_t kOnes = 0x3F803F80u;

// (a & mask) | magic in one instruction.  gfx9 VOP3 takes no literal constants, so written
// as C the compiler emits an AND and an OR with literals; here the mask comes from a
// scalar register and the magic exponent from a vector register (one constant-bus read).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(magic));
  return r;
}

struct Magic {
  uint32_t m128, m32, m8;  // bf16 pairs 128, 32 and 8 (vector registers)
};

__device__ __forceinline__ void unpack_word(uint32_t w, const Magic& mg, u32x4_t& b0, u32x4_t& b1) {
  const uint32_t w6 = w >> 6, w12 = w >> 12;
  b0[0] = and_or(w, 0x00030003u, mg.m128);    // 128 + q: inputs 0, 1
  b0[1] = and_or(w, 0x000C000Cu, mg.m32);     //  32 + q: inputs 2, 3
  b0[2] = and_or(w, 0x00300030u, mg.m8);      //   8 + q: inputs 4, 5
  b0[3] = and_or(w6, 0x00030003u, mg.m128);   // 128 + q: inputs 6, 7
  b1[0] = and_or(w6, 0x000C000Cu, mg.m32);    //  32 + q: inputs 8, 9
  b1[1] = and_or(w6, 0x00300030u, mg.m8);     //   8 + q: inputs 10, 11
  b1[2] = and_or(w12, 0x00030003u, mg.m128);  // 128 + q: inputs 12, 13
  b1[3] = and_or(w12, 0x000C000Cu, mg.m32);   //  32 + q: inputs 14, 15
}

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4_t ldg16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

template <int G, int S, int TPW>
struct Codes {
  static constexpr int GPT = 256 / G;
  u32x4_t cw[TPW][S];
  uint32_t pv[TPW][S][GPT];
};

// Raw buffer loads: one scalar resource per slice, a scalar tile offset and one per-lane
// offset that never changes, so the loop needs no vector address arithmetic.  (Buffer
// loads are also bounds-checked by the hardware against the slice size.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const uint8_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, int(bytes), 0x00020000);
}

template <int G, int S, int TPW>
__device__ __forceinline__ void load_codes(Codes<G, S, TPW>& C, const __amdgpu_buffer_rsrc_t (&rs)[S],
                                           int nb, const int (&kt)[TPW], int KB, int NG,
                                           uint32_t po, uint32_t lane_code, uint32_t lane_par) {
  constexpr int GPT = 256 / G;
#pragma unroll
  for (int j = 0; j < S; ++j) {
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp) {
      const uint32_t tile = uint32_t(nb * KB + kt[tp]) * kTileBytes;
      C.cw[tp][j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs[j], lane_code, tile, 0));
      const uint32_t par = po + uint32_t(nb * NG + kt[tp] * GPT) * 64;
#pragma unroll
      for (int gi = 0; gi < GPT; ++gi)
        C.pv[tp][j][gi] = __builtin_amdgcn_raw_buffer_load_b32(rs[j], lane_par, par + gi * 64, 0);
    }
  }
}

// At most 8 waves (two per SIMD), so a wave has 256 registers: room for its stationary
// A operand and seeds plus three buffers of codes and params without any spill (a spill
// would wait on the in-order load counter behind the prefetched loads).
template <int G, int S, int NA, int TPW>
__global__ __launch_bounds__(512) void decode_stream_kernel(
    const uint8_t* __restrict__ packed, int N, int K, int KB, int NG, int NB, uint64_t ss,
    uint64_t po, const void* __restrict__ x, int T, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, void* __restrict__ y, int y_bf16) {
  constexpr int GPT = 256 / G, WPG = G / 64;
  __shared__ f32x4_t red[2][kMaxWaves][64];
  const int NW = blockDim.x >> 6;
  // the wave index is uniform: telling the compiler keeps tile addresses in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane & 15, c = lane >> 4;
  const int step = gridDim.x;

  int kt[TPW];
  bool live[TPW];
#pragma unroll
  for (int tp = 0; tp < TPW; ++tp) {
    const int t = wave + NW * tp;
    live[tp] = t < KB;
    kt[tp] = live[tp] ? t : 0;
  }

  // ---- 1. loads that depend on nothing: this wave's activations (row r = token r; rows
  // past T repeat the last token and are never stored).
  const int xr = min(r, T - 1);
  u32x4_t Araw[TPW][4][2][NA];
#pragma unroll
  for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t k = size_t(kt[tp]) * 256 + 64 * i + 16 * c;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < NA; ++q) {
          const uint8_t* p = static_cast<const uint8_t*>(x) + (size_t(xr) * K + k + 8 * h) * (2 * NA) + 16 * q;
          Araw[tp][i][h][q] = ldg16(p);
        }
    }
  Codes<G, S, TPW> c0, c1, c2;
  u32x4_t A[TPW][4][2][NA];

  // ---- 2. routing data through the scalar cache (uniform addresses; its own counter, so
  // nothing here waits on the vector loads above): slices any token needs (jmax) and, per
  // row of this lane, its budget.
  int off[S + 1];
#pragma unroll
  for (int j = 0; j <= S; ++j) off[j] = offsets[j];
  int pm[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) pm[i] = perm[min(i, T - 1)];
  int jmax = 1;
#pragma unroll
  for (int j = 1; j < S; ++j)
    if (off[j] <= T - 1) jmax = j + 1;
  // one buffer resource per slice; a slice no token needs points at slice 0 (cached)
  __amdgpu_buffer_rsrc_t rs[S];
#pragma unroll
  for (int j = 0; j < S; ++j) rs[j] = slice_rsrc(packed + uint64_t(j < jmax ? j : 0) * ss, uint32_t(ss));
  const uint32_t lane_code = 16u * lane, lane_par = 4u * (lane & 15);
  int bud[4] = {0, 0, 0, 0};  // budget of token 4c + v
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int tok = pm[i];
    int b = 1;
#pragma unroll
    for (int j = 1; j < S; ++j)
      if (off[j] <= i) b = j + 1;
    if (i >= T) b = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (tok == 4 * c + v && b > 0) bud[v] = b;
  }

  // ---- 3. A operands (float32 inputs split into bf16 high and low parts) and the seeds
  // -sum x*o, sum x per group.  Computed inside the streaming loop, after the first weight
  // loads have been issued (see below).
  const u32x4_t bneg0{kNeg128, kNeg32, kNeg8, kNeg128};
  const u32x4_t bneg1{kNeg32, kNeg8, kNeg128, kNeg32};
  const u32x4_t ones{kOnes, kOnes, kOnes, kOnes};
  f32x4_t gnb[TPW][GPT], gxs[TPW][GPT];
  // bf16 activations are used straight from the load registers (no copy, so nothing
  // waits on them before the loop); float32 ones are split once into A.
  auto aop = [&](int tp, int i, int h, int pa) -> const u32x4_t& {
    return NA == 1 ? Araw[tp][i][h][0] : A[tp][i][h][pa];
  };
  auto setup_a = [&]() {
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (NA == 1) {
            // used in place
          } else {
            const u32x4_t q0 = Araw[tp][i][h][0], q1 = Araw[tp][i][h][NA - 1];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              const float v0 = __uint_as_float(d < 2 ? q0[2 * d] : q1[2 * d - 4]);
              const float v1 = __uint_as_float(d < 2 ? q0[2 * d + 1] : q1[2 * d - 3]);
              const uint32_t h0 = bf16_bits_rne(v0), h1 = bf16_bits_rne(v1);
              const uint32_t l0 = bf16_bits_rne(v0 - bf16_bits_to_float(h0));
              const uint32_t l1 = bf16_bits_rne(v1 - bf16_bits_to_float(h1));
              A[tp][i][h][0][d] = h0 | (h1 << 16);
              A[tp][i][h][NA - 1][d] = l0 | (l1 << 16);
            }
          }
        }
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
            nb4 = mfma(aop(tp, i, 0, pa), bneg0, nb4);
            nb4 = mfma(aop(tp, i, 1, pa), bneg1, nb4);
            xs4 = mfma(aop(tp, i, 0, pa), ones, xs4);
            xs4 = mfma(aop(tp, i, 1, pa), ones, xs4);
          }
        gnb[tp][gi] = nb4;
        gxs[tp][gi] = xs4;
      }
  };

  // ---- stream the row blocks
  const Magic mg{0x43004300u, 0x42004200u, 0x41004100u};
  auto process = [&](const Codes<G, S, TPW>& C, int nb, int buf) {
    // Per group, the (slice, tile) MFMA chains are independent: issue them interleaved so
    // the matrix pipeline never waits on one chain, then run all their epilogues.
    f32x4_t acc[S];
#pragma unroll
    for (int j = 0; j < S; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      f32x4_t P[S][TPW];
#pragma unroll
      for (int j = 0; j < S; ++j)
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) P[j][tp] = gnb[tp][gi];
#pragma unroll
      for (int ii = 0; ii < WPG; ++ii) {
        const int i = gi * WPG + ii;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int j = 0; j < S; ++j) {
            if (j < jmax) {
#pragma unroll
              for (int tp = 0; tp < TPW; ++tp) {
                u32x4_t b0, b1;
                unpack_word(C.cw[tp][j][i], mg, b0, b1);
#pragma unroll
                for (int pa = 0; pa < NA; ++pa) P[j][tp] = mfma(aop(tp, i, h, pa), h ? b1 : b0, P[j][tp]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < S; ++j) {
        if (j < jmax) {
#pragma unroll
          for (int tp = 0; tp < TPW; ++tp) {
            if (!live[tp]) continue;  // a wave without this tile (uniform); its loads were redirects
            const uint32_t pv = C.pv[tp][j][gi];
            const float s = __half2float(__ushort_as_half(uint16_t(pv & 0xFFFFu)));
            const float z = __half2float(__ushort_as_half(uint16_t(pv >> 16)));
#pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[j][v] = fmaf(s, P[j][tp][v], fmaf(z, gxs[tp][gi][v], acc[j][v]));
          }
        }
      }
    }
    f32x4_t out{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < S; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (j < bud[v]) out[v] += acc[j][v];
    red[buf][wave][lane] = out;
    __syncthreads();
    // one output per thread of the first four waves (the workgroup has at least four), so
    // every row block issues a fixed number of stores and the load waits stay exact
    if (threadIdx.x < 256) {
      const int t = threadIdx.x;
      const int p = t >> 4, n16 = t & 15;
      const int ln = 16 * (p >> 2) + n16, v = p & 3;
      float sum = 0.f;
      for (int w = 0; w < NW; ++w) sum += red[buf][w][ln][v];
      const int n = nb * 16 + n16;
      if (p < T && n < N) {
        const size_t idx = size_t(p) * N + n;
        if (y_bf16)
          reinterpret_cast<uint16_t*>(y)[idx] = uint16_t(bf16_bits_rne(sum));
        else
          reinterpret_cast<float*>(y)[idx] = sum;
      }
    }
  };

  // Three register buffers; step m loads row block m + 2 into buffer (m + 2) % 3 and then
  // multiplies row block m from buffer m % 3, so two row blocks are always in flight.
  // There is no prologue: steps -2 and -1 only load, and the seeds are computed once,
  // right after the first row block's loads are out.  Every path into the loop header therefore carries the
  // same pending loads, which keeps the compiler's waits on the in-order load counter
  // exact.  A load past the end re-reads the workgroup's first row block (cached), so
  // every load is unconditional.
  const int rb0 = blockIdx.x;
  auto nbl = [&](int m) { const int n = rb0 + m * step; return n < NB ? n : rb0; };
  int buf = 0;
  bool first = true;
  for (int m0 = -2;; m0 += 3) {
    load_codes(c0, rs, nbl(m0 + 2), kt, KB, NG, uint32_t(po), lane_code, lane_par);
    if (first) {  // seeds while the first row block is in flight (no loads in here)
      setup_a();
      first = false;
    }
    if (m0 >= 0) {
      process(c1, rb0 + m0 * step, buf);
      buf ^= 1;
      if (rb0 + (m0 + 1) * step >= NB) break;
    }
    load_codes(c1, rs, nbl(m0 + 3), kt, KB, NG, uint32_t(po), lane_code, lane_par);
    if (m0 + 1 >= 0) {
      process(c2, rb0 + (m0 + 1) * step, buf);
      buf ^= 1;
      if (rb0 + (m0 + 2) * step >= NB) break;
    }
    load_codes(c2, rs, nbl(m0 + 4), kt, KB, NG, uint32_t(po), lane_code, lane_par);
    process(c0, rb0 + (m0 + 2) * step, buf);
    buf ^= 1;
    if (rb0 + (m0 + 3) * step >= NB) break;
  }
}

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

template <int G, int S, int NA, int TPW>
hipError_t launch_gsn(const mbq_desc& d, const void* packed, int32_t t, const void* x,
                      const int32_t* perm, const int32_t* offsets, void* y, bool y_bf16,
                      hipStream_t stream) {
  const int nw = std::max(4, (d.k_tiles + TPW - 1) / TPW);  // >= 4 waves: see the store step
  const int grid = std::min(d.row_blocks, cu_count());
  hipLaunchKernelGGL((decode_stream_kernel<G, S, NA, TPW>), dim3(grid), dim3(64 * nw), 0, stream,
                     static_cast<const uint8_t*>(packed), d.n, d.k, d.k_tiles, d.groups_padded,
                     d.row_blocks, d.slice_stride, d.params_offset, x, t, perm, offsets, y,
                     int(y_bf16));
  return hipGetLastError();
}

template <int G, int NA, int TPW>
hipError_t launch_gn(const mbq_desc& d, const void* packed, int32_t t, const void* x,
                     const int32_t* perm, const int32_t* offsets, void* y, bool y_bf16,
                     hipStream_t stream) {
  switch (d.slices) {
    case 1: return launch_gsn<G, 1, NA, TPW>(d, packed, t, x, perm, offsets, y, y_bf16, stream);
    case 2: return launch_gsn<G, 2, NA, TPW>(d, packed, t, x, perm, offsets, y, y_bf16, stream);
    case 3: return launch_gsn<G, 3, NA, TPW>(d, packed, t, x, perm, offsets, y, y_bf16, stream);
    default: return launch_gsn<G, 4, NA, TPW>(d, packed, t, x, perm, offsets, y, y_bf16, stream);
  }
}

template <int G>
hipError_t launch_g(const mbq_desc& d, const void* packed, int32_t t, const void* x, bool x_bf16,
                    const int32_t* perm, const int32_t* offsets, void* y, bool y_bf16,
                    hipStream_t stream) {
  const bool two = d.k_tiles > kMaxWaves;  // 9..16 tiles: two per wave
  if (x_bf16)
    return two ? launch_gn<G, 1, 2>(d, packed, t, x, perm, offsets, y, y_bf16, stream)
               : launch_gn<G, 1, 1>(d, packed, t, x, perm, offsets, y, y_bf16, stream);
  return two ? launch_gn<G, 2, 2>(d, packed, t, x, perm, offsets, y, y_bf16, stream)
             : launch_gn<G, 2, 1>(d, packed, t, x, perm, offsets, y, y_bf16, stream);
}

}  // namespace

bool decode_stream_supported(const mbq_desc& d, int32_t t) {
  // buffer offsets are 32-bit: a slice must stay below 4 GiB
  return t >= 1 && t <= 16 && d.k_tiles <= 2 * kMaxWaves && d.slice_stride < (uint64_t(1) << 32);
}

hipError_t launch_decode_stream(const mbq_desc& d, const void* packed, int32_t t, const void* x,
                                bool x_bf16, const int32_t* perm, const int32_t* offsets,
                                void* y, bool y_bf16, hipStream_t stream) {
  switch (d.group) {
    case 64: return launch_g<64>(d, packed, t, x, x_bf16, perm, offsets, y, y_bf16, stream);
    case 128: return launch_g<128>(d, packed, t, x, x_bf16, perm, offsets, y, y_bf16, stream);
    default: return launch_g<256>(d, packed, t, x, x_bf16, perm, offsets, y, y_bf16, stream);
  }
}

}  // namespace mbq
