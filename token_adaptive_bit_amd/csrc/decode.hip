// Routed decode linear (T <= 64): y_t = x_t . (sum_{j <= b(t)} deq(Q_j))^T.
//
// MoBiQuant explainer (gist.science, English), sections 2.A and 3: every token rebuilds
// its own precision from the shared slices, and a kernel that fetches only the slices in
// use turns fewer bits into fewer bytes.  Decode is bound by HBM: this kernel streams each
// needed slice of the packed blob exactly once, in coalesced 1 KiB tile loads, never
// materializes a dequantized weight, and is a single launch with no workspace.
//
// Arithmetic.  For one (slice j, row n, group g) with stored half scale s and zero z,
//   sum_{k in g} x_k (z + s q_k) = s * P + z * X_g,   P = sum_k x_k q_k,  X_g = sum_k x_k.
// P comes from MFMA 16x16x32 bf16 (float32 accumulate) with tokens as the A operand and the
// raw codes as the B operand.  Even inputs sit in the low half-word of a code word and odd
// inputs in the high half-word, so one AND-OR against a magic exponent turns two codes
// into the bf16 pair (o + q_even, o + q_odd) with o = 128, 32 or 8 (three codes per
// half-word need no shift), in the natural input order of x.  The o-terms and X_g come
// from the same A operand multiplied by constant B operands (-o and 1), so the group's
// accumulator simply starts at -sum_k x_k o_k.  Products are exact in float32; the only
// rounding is the float32 accumulation.  float32 activations run as bf16 high + low parts.
//
// Work split.  A workgroup owns RB row blocks (16 rows each) and all of K; its NW waves
// take contiguous ranges of k tiles.  Each wave double-buffers a whole k tile (codes and
// params of every needed slice and row block, plus the A operand of every token block),
// so the next tile's loads are in flight while the current one is multiplied.  The
// waves' partial sums meet in LDS; per-token slice masks are applied there (tokens are
// sorted by budget, so slice j counts for sorted position p iff p >= offsets[j]).
#include "mbq_internal.h"

namespace mbq {
namespace {

constexpr int kMaxWaves = 8;
constexpr uint32_t kNeg128 = 0xC300C300u, kNeg32 = 0xC200C200u, kNeg8 = 0xC100C100u;
constexpr uint32_t kOnes = 0x3F803F80u;

__device__ __forceinline__ void unpack_word(uint32_t w, u32x4_t& b0, u32x4_t& b1) {
  const uint32_t w6 = w >> 6, w12 = w >> 12;
  b0[0] = (w & 0x00030003u) | 0x43004300u;    // 128 + q: inputs 0, 1
  b0[1] = (w & 0x000C000Cu) | 0x42004200u;    //  32 + q: inputs 2, 3
  b0[2] = (w & 0x00300030u) | 0x41004100u;    //   8 + q: inputs 4, 5
  b0[3] = (w6 & 0x00030003u) | 0x43004300u;   // 128 + q: inputs 6, 7
  b1[0] = (w6 & 0x000C000Cu) | 0x42004200u;   //  32 + q: inputs 8, 9
  b1[1] = (w6 & 0x00300030u) | 0x41004100u;   //   8 + q: inputs 10, 11
  b1[2] = (w12 & 0x00030003u) | 0x43004300u;  // 128 + q: inputs 12, 13
  b1[3] = (w12 & 0x000C000Cu) | 0x42004200u;  //  32 + q: inputs 14, 15
}

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4_t ldg16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// One k tile's worth of loads for one wave.  G32: groups of 32 inputs (8 per tile).
template <int TB, int RB, int SMAX, bool XF32, bool G32>
struct Bundle {
  static constexpr int GPT = G32 ? 8 : 4;
  u32x4_t cw[SMAX][RB];                 // 64 codes per lane per (slice, row block)
  uint32_t pv[SMAX][RB][GPT];           // (scale, zero) per group in the tile
  u32x4_t a[TB][XF32 ? 16 : 8];         // A: word i, half h -> [2i + h] (bf16) or raw f32
};

template <int TB, int RB, int SMAX, bool XF32, bool G32>
__device__ __forceinline__ void load_bundle(Bundle<TB, RB, SMAX, XF32, G32>& B, int kt,
                                            const uint8_t* __restrict__ packed, int K, int KB, int NG,
                                            int NB, int gpt, int nb0, int jmax,
                                            uint64_t slice_stride, uint64_t params_offset,
                                            const char* const (&xrow)[TB], const bool (&xlive)[TB],
                                            int lane) {
  const int r = lane & 15, c = lane >> 4;
#pragma unroll
  for (int j = 0; j < SMAX; ++j) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int nb = nb0 + rb;
      if (j < jmax && nb < NB) {
        const uint8_t* sl = packed + uint64_t(j) * slice_stride;
        B.cw[j][rb] = ldg16(sl + (size_t(nb) * KB + kt) * kTileBytes + 16 * lane);
        const uint8_t* pp = sl + params_offset + ((size_t(nb) * NG + size_t(kt) * gpt) * 16 + r) * 4;
#pragma unroll
        for (int gi = 0; gi < B.GPT; ++gi)
          B.pv[j][rb][gi] = (gi < gpt) ? *reinterpret_cast<const uint32_t*>(pp + gi * 64) : 0u;
      } else {
        B.cw[j][rb] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int gi = 0; gi < B.GPT; ++gi) B.pv[j][rb][gi] = 0u;
      }
    }
  }
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    constexpr int kEl = XF32 ? 4 : 2;  // bytes per activation
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t k = size_t(kt) * 256 + 64 * i + 16 * c;
      const char* p = xrow[tb] + k * kEl;
      // K is a multiple of 16: a lane's 16 inputs lie wholly inside or wholly past the row
      const bool in = xlive[tb] && k < size_t(K);
      if (XF32) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          B.a[tb][4 * i + q] = in ? ldg16(p + 16 * q) : u32x4_t{0u, 0u, 0u, 0u};
      } else {
        B.a[tb][2 * i] = in ? ldg16(p) : u32x4_t{0u, 0u, 0u, 0u};
        B.a[tb][2 * i + 1] = in ? ldg16(p + 16) : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }
}

// float32 x -> (bf16 high, bf16 low) operands for word i, half h (8 inputs).
__device__ __forceinline__ void split_f32(const u32x4_t& q0, const u32x4_t& q1, u32x4_t& hi,
                                          u32x4_t& lo) {
  float v[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = __uint_as_float(q0[e]);
    v[4 + e] = __uint_as_float(q1[e]);
  }
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t h0 = bf16_bits_rne(v[2 * d]), h1 = bf16_bits_rne(v[2 * d + 1]);
    const uint32_t l0 = bf16_bits_rne(v[2 * d] - bf16_bits_to_float(h0));
    const uint32_t l1 = bf16_bits_rne(v[2 * d + 1] - bf16_bits_to_float(h1));
    hi[d] = h0 | (h1 << 16);
    lo[d] = l0 | (l1 << 16);
  }
}

template <int TB, int RB, int SMAX, bool XF32, bool G32>
__device__ __forceinline__ void compute_bundle(const Bundle<TB, RB, SMAX, XF32, G32>& B, int wpg,
                                               int jmax, const int (&jlim)[TB], int c,
                                               f32x4_t (&acc)[SMAX][TB][RB]) {
  const u32x4_t bneg0{kNeg128, kNeg32, kNeg8, kNeg128};   // -o for inputs 0..7
  const u32x4_t bneg1{kNeg32, kNeg8, kNeg128, kNeg32};    // -o for inputs 8..15
  const u32x4_t ones{kOnes, kOnes, kOnes, kOnes};
  const f32x4_t zero4{0.f, 0.f, 0.f, 0.f};
  constexpr int NA = XF32 ? 2 : 1;   // A parts: bf16 high (+ low)

  // A operands of the four words, per part
  u32x4_t A[TB][4][2][NA];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (XF32) {
          u32x4_t hi, lo;
          split_f32(B.a[tb][4 * i + 2 * h], B.a[tb][4 * i + 2 * h + 1], hi, lo);
          A[tb][i][h][0] = hi;
          A[tb][i][h][NA - 1] = lo;
        } else {
          A[tb][i][h][0] = B.a[tb][2 * i + h];
        }
      }

  f32x4_t P[SMAX][TB][RB];
  f32x4_t gxs[TB];
  if constexpr (G32) {
    // Word i holds groups 2i (lanes c = 0, 1) and 2i + 1 (c = 2, 3) of the tile: each group
    // runs the MFMAs on an A operand with the other group's lanes zeroed.
    const u32x4_t z4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int sg = 0; sg < 2; ++sg) {
        const bool mine = (c >> 1) == sg;
        u32x4_t Am[TB][2][NA];
        f32x4_t gnb[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          gnb[tb] = zero4;
          gxs[tb] = zero4;
#pragma unroll
          for (int pa = 0; pa < NA; ++pa) {
            Am[tb][0][pa] = mine ? A[tb][i][0][pa] : z4;
            Am[tb][1][pa] = mine ? A[tb][i][1][pa] : z4;
            gnb[tb] = mfma(Am[tb][0][pa], bneg0, gnb[tb]);
            gnb[tb] = mfma(Am[tb][1][pa], bneg1, gnb[tb]);
            gxs[tb] = mfma(Am[tb][0][pa], ones, gxs[tb]);
            gxs[tb] = mfma(Am[tb][1][pa], ones, gxs[tb]);
          }
        }
#pragma unroll
        for (int j = 0; j < SMAX; ++j) {
          if (j >= jmax) break;
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            u32x4_t b0, b1;
            unpack_word(B.cw[j][rb][i], b0, b1);
            const uint32_t pv = B.pv[j][rb][2 * i + sg];
            const float s = __half2float(__ushort_as_half(uint16_t(pv & 0xFFFFu)));
            const float z = __half2float(__ushort_as_half(uint16_t(pv >> 16)));
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
              if (j < jlim[tb]) {
                f32x4_t p = gnb[tb];
#pragma unroll
                for (int pa = 0; pa < NA; ++pa) {
                  p = mfma(Am[tb][0][pa], b0, p);
                  p = mfma(Am[tb][1][pa], b1, p);
                }
#pragma unroll
                for (int v = 0; v < 4; ++v)
                  acc[j][tb][rb][v] = fmaf(s, p[v], fmaf(z, gxs[tb][v], acc[j][tb][rb][v]));
              }
            }
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i % wpg == 0) {
      // group start: -sum x*o and sum x over the group's words, then seed every chain
      f32x4_t gnb[TB];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        gnb[tb] = zero4;
        gxs[tb] = zero4;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          if (i2 / wpg == i / wpg) {
#pragma unroll
            for (int pa = 0; pa < NA; ++pa) {
              gnb[tb] = mfma(A[tb][i2][0][pa], bneg0, gnb[tb]);
              gnb[tb] = mfma(A[tb][i2][1][pa], bneg1, gnb[tb]);
              gxs[tb] = mfma(A[tb][i2][0][pa], ones, gxs[tb]);
              gxs[tb] = mfma(A[tb][i2][1][pa], ones, gxs[tb]);
            }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < SMAX; ++j)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) P[j][tb][rb] = gnb[tb];
    }
#pragma unroll
    for (int j = 0; j < SMAX; ++j) {
      if (j >= jmax) break;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        u32x4_t b0, b1;
        unpack_word(B.cw[j][rb][i], b0, b1);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          if (j < jlim[tb]) {
#pragma unroll
            for (int pa = 0; pa < NA; ++pa) {
              P[j][tb][rb] = mfma(A[tb][i][0][pa], b0, P[j][tb][rb]);
              P[j][tb][rb] = mfma(A[tb][i][1][pa], b1, P[j][tb][rb]);
            }
          }
        }
      }
    }
    if (i % wpg == wpg - 1) {
      // group end: scale and zero of (slice, row) for this group
#pragma unroll
      for (int j = 0; j < SMAX; ++j) {
        if (j >= jmax) break;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const uint32_t pv = (wpg == 1) ? B.pv[j][rb][i]
                            : (wpg == 2) ? B.pv[j][rb][i >> 1] : B.pv[j][rb][0];
          const float s = __half2float(__ushort_as_half(uint16_t(pv & 0xFFFFu)));
          const float z = __half2float(__ushort_as_half(uint16_t(pv >> 16)));
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) {
            if (j < jlim[tb]) {
#pragma unroll
              for (int v = 0; v < 4; ++v)
                acc[j][tb][rb][v] = fmaf(s, P[j][tb][rb][v], fmaf(z, gxs[tb][v], acc[j][tb][rb][v]));
            }
          }
        }
      }
    }
  }
}

template <int TB, int RB, int SMAX, bool XF32, bool G32>
__global__ __launch_bounds__(512) void decode_kernel(
    const uint8_t* __restrict__ packed, int N, int K, int KB, int NG, int NB, int G,
    uint64_t slice_stride, uint64_t params_offset, const void* __restrict__ x, int T,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets, void* __restrict__ y,
    int y_bf16) {
  __shared__ f32x4_t red[kMaxWaves][RB * TB][64];
  const int NW = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, c = lane >> 4;
  const int nb0 = blockIdx.x * RB;
  const int kt0 = wave * KB / NW, kt1 = (wave + 1) * KB / NW;
  const int gpt = 256 / G, wpg = G / 64;

  // Slices each 16-token block needs (tokens sorted by budget: the block's last valid
  // token has the largest budget).  offsets[j] = #tokens with budget <= j.
  int off[SMAX + 1];
#pragma unroll
  for (int j = 0; j <= SMAX; ++j) off[j] = offsets[j];
  int jlim[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int last = min(16 * tb + 15, T - 1);
    int b = 1;
#pragma unroll
    for (int j = 1; j < SMAX; ++j)
      if (off[j] <= last) b = j + 1;
    jlim[tb] = b;
  }
  const int jmax = jlim[TB - 1];

  // A rows: sorted position 16*tb + r is original token perm[...]
  const char* xrow[TB];
  bool xlive[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int p = 16 * tb + r;
    xlive[tb] = p < T;
    const int pp = xlive[tb] ? perm[p] : 0;
    const int src = (pp >= 0 && pp < T) ? pp : 0;  // out-of-contract entries never address memory
    xrow[tb] = static_cast<const char*>(x) + size_t(src) * K * (XF32 ? 4 : 2);
  }

  f32x4_t acc[SMAX][TB][RB];
#pragma unroll
  for (int j = 0; j < SMAX; ++j)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[j][tb][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  Bundle<TB, RB, SMAX, XF32, G32> b0, b1;
  if (kt0 < kt1)
    load_bundle(b0, kt0, packed, K, KB, NG, NB, gpt, nb0, jmax, slice_stride, params_offset, xrow, xlive, lane);
  for (int kt = kt0; kt < kt1; kt += 2) {
    if (kt + 1 < kt1)
      load_bundle(b1, kt + 1, packed, K, KB, NG, NB, gpt, nb0, jmax, slice_stride, params_offset, xrow, xlive, lane);
    compute_bundle(b0, wpg, jmax, jlim, c, acc);
    if (kt + 1 < kt1) {
      if (kt + 2 < kt1)
        load_bundle(b0, kt + 2, packed, K, KB, NG, NB, gpt, nb0, jmax, slice_stride, params_offset, xrow, xlive, lane);
      compute_bundle(b1, wpg, jmax, jlim, c, acc);
    }
  }

  // Per-token slice masks, then the sum over the waves' k ranges.
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4_t o = acc[0][tb][rb];
#pragma unroll
      for (int j = 1; j < SMAX; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (16 * tb + 4 * c + v >= off[j]) o[v] += acc[j][tb][rb][v];
      red[wave][rb * TB + tb][lane] = o;
    }
  }
  __syncthreads();
  for (int slot = threadIdx.x; slot < RB * TB * 64; slot += blockDim.x) {
    const int rbtb = slot >> 6, ln = slot & 63;
    f32x4_t o = red[0][rbtb][ln];
    for (int w = 1; w < NW; ++w) {
      const f32x4_t q = red[w][rbtb][ln];
#pragma unroll
      for (int v = 0; v < 4; ++v) o[v] += q[v];
    }
    const int rb = rbtb / TB, tb = rbtb % TB;
    const int n = (nb0 + rb) * 16 + (ln & 15);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int p = 16 * tb + 4 * (ln >> 4) + v;
      const int tok = p < T ? perm[p] : -1;
      if (tok >= 0 && tok < T && n < N) {
        const size_t idx = size_t(tok) * N + n;
        if (y_bf16)
          reinterpret_cast<uint16_t*>(y)[idx] = uint16_t(bf16_bits_rne(o[v]));
        else
          reinterpret_cast<float*>(y)[idx] = o[v];
      }
    }
  }
}

// Waves per workgroup: split the k tiles evenly, at least two tiles per wave.
int waves_for(int KB) {
  for (int nw = kMaxWaves; nw >= 2; --nw)
    if (KB % nw == 0 && KB / nw >= 2) return nw;
  return std::max(1, std::min(kMaxWaves, KB / 2));
}

template <int TB, int RB, int SMAX, bool XF32>
hipError_t launch_k(const mbq_desc& d, const void* packed, int32_t t, const void* x,
                    const int32_t* perm, const int32_t* offsets, void* y, bool y_bf16,
                    hipStream_t stream) {
  const int nw = waves_for(d.k_tiles);
  dim3 grid((d.row_blocks + RB - 1) / RB), block(64 * nw);
  if (d.group == 32)
    hipLaunchKernelGGL((decode_kernel<TB, RB, SMAX, XF32, true>), grid, block, 0, stream,
                       static_cast<const uint8_t*>(packed), d.n, d.k, d.k_tiles, d.groups_padded,
                       d.row_blocks, d.group, d.slice_stride, d.params_offset, x, t, perm,
                       offsets, y, int(y_bf16));
  else
    hipLaunchKernelGGL((decode_kernel<TB, RB, SMAX, XF32, false>), grid, block, 0, stream,
                       static_cast<const uint8_t*>(packed), d.n, d.k, d.k_tiles, d.groups_padded,
                       d.row_blocks, d.group, d.slice_stride, d.params_offset, x, t, perm,
                       offsets, y, int(y_bf16));
  return hipGetLastError();
}

template <int SMAX, bool XF32>
hipError_t launch_s(const mbq_desc& d, const void* packed, int32_t t, const void* x,
                    const int32_t* perm, const int32_t* offsets, void* y, bool y_bf16,
                    hipStream_t stream) {
  switch ((t + 15) / 16) {
    case 1: return launch_k<1, XF32 ? 1 : 2, SMAX, XF32>(d, packed, t, x, perm, offsets, y, y_bf16, stream);
    case 2: return launch_k<2, XF32 ? 1 : 2, SMAX, XF32>(d, packed, t, x, perm, offsets, y, y_bf16, stream);
    case 3: return launch_k<3, 1, SMAX, XF32>(d, packed, t, x, perm, offsets, y, y_bf16, stream);
    default: return launch_k<4, 1, SMAX, XF32>(d, packed, t, x, perm, offsets, y, y_bf16, stream);
  }
}

}  // namespace

size_t decode_workspace(const mbq_desc&, int32_t, bool) { return 0; }

hipError_t launch_decode(const mbq_desc& d, const void* packed, int32_t t, const void* x,
                         bool x_bf16, const int32_t* perm, const int32_t* offsets, void* y,
                         bool y_bf16, void*, hipStream_t stream) {
  const bool f32 = !x_bf16;
  switch (d.slices) {
    case 1: return f32 ? launch_s<1, true>(d, packed, t, x, perm, offsets, y, y_bf16, stream)
                       : launch_s<1, false>(d, packed, t, x, perm, offsets, y, y_bf16, stream);
    case 2: return f32 ? launch_s<2, true>(d, packed, t, x, perm, offsets, y, y_bf16, stream)
                       : launch_s<2, false>(d, packed, t, x, perm, offsets, y, y_bf16, stream);
    case 3: return f32 ? launch_s<3, true>(d, packed, t, x, perm, offsets, y, y_bf16, stream)
                       : launch_s<3, false>(d, packed, t, x, perm, offsets, y, y_bf16, stream);
    default: return f32 ? launch_s<4, true>(d, packed, t, x, perm, offsets, y, y_bf16, stream)
                        : launch_s<4, false>(d, packed, t, x, perm, offsets, y, y_bf16, stream);
  }
}

}  // namespace mbq
