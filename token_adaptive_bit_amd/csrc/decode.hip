// Routed decode linear (T <= 64): y_t = x_t . (sum_{j <= b(t)} deq(Q_j))^T.
//
// MoBiQuant explainer (gist.science, English), sections 2.A and 3: every token rebuilds
// its own precision from the shared slices, and a kernel that fetches only the slices in
// use turns fewer bits into fewer bytes.  Decode is bound by HBM: the kernel streams each
// needed slice of the packed blob exactly once, in coalesced 1 KiB tile loads, and never
// materializes a dequantized weight.
//
// Arithmetic.  For one (slice j, row n, group g) with stored half scale s and zero z,
//   sum_{k in g} x_k (z + s q_k) = s * P + z * X_g,   P = sum_k x_k q_k,  X_g = sum_k x_k.
// P is an MFMA (16x16x32 bf16, float32 accumulate) with the tokens as the A operand and
// the raw codes as the B operand: a code q becomes the exact bfloat16 value o + q with one
// AND-OR against a magic exponent (o = 128, 32 or 8 depending on the bit position inside
// the 16-bit half, so three codes per half need no shift).  The o-term is cancelled by
// starting the group's accumulator at -sum_k x_k o_k, precomputed per (token, group).
// Products are exact, so the only rounding is the float32 accumulation.
//
// The pre-pass writes x in sorted (regrouped) token order, zero-padded to 16-token blocks
// and to 256-input tiles, with the inputs of every 16-input chunk interleaved as
// (e, e+8) pairs to match the code pairs the AND-OR produces; float32 inputs are split
// into bfloat16 high and low parts that run as two MFMAs.
#include "mbq_internal.h"

namespace mbq {
namespace {

constexpr int kNW = 4;  // waves per workgroup (split K)

__device__ __forceinline__ float group_offset(int e) {
  // bias of the magic value at position e (0..15) of a 16-input chunk
  const int s = e & 7;
  return (s % 3 == 0) ? 128.f : ((s % 3 == 1) ? 32.f : 8.f);
}

// One thread per (sorted token, 16-input chunk).  The G/16 chunks of a group sit in
// consecutive lanes and are reduced with butterflies.
template <bool XBF16, bool SPLIT>
__global__ __launch_bounds__(256) void xprep_kernel(const void* __restrict__ x, int T, int K,
                                                    int Kp, int T16, int G,
                                                    const int32_t* __restrict__ perm,
                                                    uint16_t* __restrict__ xh,
                                                    uint16_t* __restrict__ xl,
                                                    float* __restrict__ xs,
                                                    float* __restrict__ nbias) {
  const int chunks = Kp / 16;
  const int total = T16 * chunks;
  const int tid = blockIdx.x * 256 + threadIdx.x;
  const bool live = tid < total;
  const int i = live ? tid / chunks : 0;
  const int ch = live ? tid % chunks : 0;
  const int src = (live && i < T) ? perm[i] : -1;
  const int k0 = ch * 16;
  float v[16];
#pragma unroll
  for (int e = 0; e < 16; ++e)
    v[e] = (src >= 0 && k0 + e < K) ? load_x(x, size_t(src) * K + k0 + e, XBF16) : 0.f;
  uint32_t hb[16], lb[16];
  float sum = 0.f, bias = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    hb[e] = bf16_bits_rne(v[e]);
    float xt = bf16_bits_to_float(hb[e]);
    if (SPLIT) {
      lb[e] = bf16_bits_rne(v[e] - xt);
      xt += bf16_bits_to_float(lb[e]);
    } else {
      lb[e] = 0;
    }
    sum += xt;
    bias = fmaf(xt, group_offset(e), bias);
  }
  if (live) {
    u32x4_t h0, h1, l0, l1;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      h0[s] = hb[s] | (hb[s + 8] << 16);
      h1[s] = hb[s + 4] | (hb[s + 12] << 16);
      l0[s] = lb[s] | (lb[s + 8] << 16);
      l1[s] = lb[s + 4] | (lb[s + 12] << 16);
    }
    u32x4_t* dh = reinterpret_cast<u32x4_t*>(xh + size_t(i) * Kp + k0);
    dh[0] = h0;
    dh[1] = h1;
    if (SPLIT) {
      u32x4_t* dl = reinterpret_cast<u32x4_t*>(xl + size_t(i) * Kp + k0);
      dl[0] = l0;
      dl[1] = l1;
    }
  }
  const int cpg = G / 16;  // chunks per group: 4, 8 or 16
  for (int o = 1; o < cpg; o <<= 1) {
    sum += __shfl_xor(sum, o);
    bias += __shfl_xor(bias, o);
  }
  if (live && (ch % cpg) == 0) {
    const int g = ch / cpg;
    xs[size_t(g) * T16 + i] = sum;
    nbias[size_t(g) * T16 + i] = -bias;
  }
}

__device__ __forceinline__ void unpack_word(uint32_t w, u32x4_t& b0, u32x4_t& b1) {
  const uint32_t w6 = w >> 6, w12 = w >> 12;
  b0[0] = (w & 0x00030003u) | 0x43004300u;    // 128 + q, codes e = 0 / 8
  b0[1] = (w & 0x000C000Cu) | 0x42004200u;    //  32 + q, codes 1 / 9
  b0[2] = (w & 0x00300030u) | 0x41004100u;    //   8 + q, codes 2 / 10
  b0[3] = (w6 & 0x00030003u) | 0x43004300u;   // 128 + q, codes 3 / 11
  b1[0] = (w6 & 0x000C000Cu) | 0x42004200u;   //  32 + q, codes 4 / 12
  b1[1] = (w6 & 0x00300030u) | 0x41004100u;   //   8 + q, codes 5 / 13
  b1[2] = (w12 & 0x00030003u) | 0x43004300u;  // 128 + q, codes 6 / 14
  b1[3] = (w12 & 0x000C000Cu) | 0x42004200u;  //  32 + q, codes 7 / 15
}

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Workgroup = kNW waves = RB row blocks (16 rows each) x all of K; wave w takes k tiles
// w, w + kNW, ...  Partial results meet in LDS at the end.
template <int TB, int RB, int SMAX, bool SPLIT>
__global__ __launch_bounds__(256) void decode_kernel(
    const uint8_t* __restrict__ packed, int N, int KB, int NG, int NB, int G,
    uint64_t slice_stride, uint64_t params_offset, const uint16_t* __restrict__ xh,
    const uint16_t* __restrict__ xl, const float* __restrict__ xs,
    const float* __restrict__ nbias, int T, int T16, int Kp,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets, void* __restrict__ y,
    int y_bf16) {
  __shared__ f32x4_t red[kNW][RB * TB][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, c = lane >> 4;
  const int nb0 = blockIdx.x * RB;
  const int wpg = G / 64;  // words per group: 1, 2 or 4

  // Slices each 16-token block needs: tokens are sorted by budget, so the block's last
  // valid token has the largest budget.  offsets[j] = #tokens with budget <= j.
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

  f32x4_t acc[SMAX][TB][RB];
#pragma unroll
  for (int j = 0; j < SMAX; ++j)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[j][tb][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int kb = wave; kb < KB; kb += kNW) {
    u32x4_t wv[SMAX][RB];
#pragma unroll
    for (int j = 0; j < SMAX; ++j)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int nb = nb0 + rb;
        if (j < jmax && nb < NB)
          wv[j][rb] = *reinterpret_cast<const u32x4_t*>(packed + uint64_t(j) * slice_stride +
                                                        (size_t(nb) * KB + kb) * kTileBytes + 16 * lane);
        else
          wv[j][rb] = u32x4_t{0u, 0u, 0u, 0u};
      }
    f32x4_t P[SMAX][TB][RB];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = (kb * 4 + i) / wpg;
      if (i % wpg == 0) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          const f32x4_t nbv = *reinterpret_cast<const f32x4_t*>(nbias + size_t(g) * T16 + 16 * tb + 4 * c);
#pragma unroll
          for (int j = 0; j < SMAX; ++j)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) P[j][tb][rb] = nbv;
        }
      }
      u32x4_t ah0[TB], ah1[TB], al0[TB], al1[TB];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const size_t base = size_t(16 * tb + r) * Kp + size_t(kb) * 256 + 64 * i + 16 * c;
        const u32x4_t* ph = reinterpret_cast<const u32x4_t*>(xh + base);
        ah0[tb] = ph[0];
        ah1[tb] = ph[1];
        if (SPLIT) {
          const u32x4_t* pl = reinterpret_cast<const u32x4_t*>(xl + base);
          al0[tb] = pl[0];
          al1[tb] = pl[1];
        }
      }
#pragma unroll
      for (int j = 0; j < SMAX; ++j) {
        if (j >= jmax) break;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          u32x4_t b0, b1;
          unpack_word(wv[j][rb][i], b0, b1);
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) {
            if (j < jlim[tb]) {
              P[j][tb][rb] = mfma(ah0[tb], b0, P[j][tb][rb]);
              P[j][tb][rb] = mfma(ah1[tb], b1, P[j][tb][rb]);
              if (SPLIT) {
                P[j][tb][rb] = mfma(al0[tb], b0, P[j][tb][rb]);
                P[j][tb][rb] = mfma(al1[tb], b1, P[j][tb][rb]);
              }
            }
          }
        }
      }
      if (i % wpg == wpg - 1) {
        f32x4_t xsv[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
          xsv[tb] = *reinterpret_cast<const f32x4_t*>(xs + size_t(g) * T16 + 16 * tb + 4 * c);
#pragma unroll
        for (int j = 0; j < SMAX; ++j) {
          if (j >= jmax) break;
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const int nb = nb0 + rb;
            uint32_t pv = 0;
            if (nb < NB)
              pv = *reinterpret_cast<const uint32_t*>(packed + uint64_t(j) * slice_stride + params_offset +
                                                      ((size_t(nb) * NG + g) * 16 + r) * 4);
            const float s = __half2float(__ushort_as_half(uint16_t(pv & 0xFFFFu)));
            const float z = __half2float(__ushort_as_half(uint16_t(pv >> 16)));
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
              if (j < jlim[tb]) {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                  acc[j][tb][rb][v] = fmaf(s, P[j][tb][rb][v], fmaf(z, xsv[tb][v], acc[j][tb][rb][v]));
              }
            }
          }
        }
      }
    }
  }

  // Per-token slice masks (slice j counts for sorted position p iff p >= offsets[j]),
  // then the split-K sum across waves.
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
  for (int slot = threadIdx.x; slot < RB * TB * 64; slot += 256) {
    const int rbtb = slot >> 6, ln = slot & 63;
    f32x4_t o = red[0][rbtb][ln];
#pragma unroll
    for (int w = 1; w < kNW; ++w) {
      const f32x4_t q = red[w][rbtb][ln];
#pragma unroll
      for (int v = 0; v < 4; ++v) o[v] += q[v];
    }
    const int rb = rbtb / TB, tb = rbtb % TB;
    const int n = (nb0 + rb) * 16 + (ln & 15);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int p = 16 * tb + 4 * (ln >> 4) + v;
      if (p < T && n < N) {
        const size_t idx = size_t(perm[p]) * N + n;
        if (y_bf16)
          reinterpret_cast<uint16_t*>(y)[idx] = uint16_t(bf16_bits_rne(o[v]));
        else
          reinterpret_cast<float*>(y)[idx] = o[v];
      }
    }
  }
}

struct DecodeWs {
  uint16_t* xh;
  uint16_t* xl;
  float* xs;
  float* nbias;
  size_t bytes;
};

DecodeWs carve(const mbq_desc& d, int32_t t, bool x_bf16, void* base) {
  const size_t T16 = size_t((t + 15) / 16) * 16;
  const size_t Kp = size_t(d.k_tiles) * 256;
  auto a256 = [](size_t v) { return (v + 255) & ~size_t(255); };
  const size_t xbytes = a256(T16 * Kp * 2);
  const size_t sbytes = a256(T16 * size_t(d.groups_padded) * 4);
  char* p = static_cast<char*>(base);
  DecodeWs w;
  w.xh = reinterpret_cast<uint16_t*>(p);
  w.xl = x_bf16 ? nullptr : reinterpret_cast<uint16_t*>(p + xbytes);
  const size_t xtot = x_bf16 ? xbytes : 2 * xbytes;
  w.xs = reinterpret_cast<float*>(p + xtot);
  w.nbias = reinterpret_cast<float*>(p + xtot + sbytes);
  w.bytes = xtot + 2 * sbytes;
  return w;
}

template <int TB, int SMAX, bool SPLIT>
hipError_t launch_tb(const mbq_desc& d, const void* packed, int32_t t, const DecodeWs& w,
                     const int32_t* perm, const int32_t* offsets, void* y, bool y_bf16,
                     hipStream_t stream) {
  constexpr int RB = (TB <= 2) ? 2 : 1;
  const int T16 = ((t + 15) / 16) * 16;
  dim3 grid((d.row_blocks + RB - 1) / RB), block(256);
  hipLaunchKernelGGL((decode_kernel<TB, RB, SMAX, SPLIT>), grid, block, 0, stream,
                     static_cast<const uint8_t*>(packed), d.n, d.k_tiles, d.groups_padded,
                     d.row_blocks, d.group, d.slice_stride, d.params_offset, w.xh, w.xl, w.xs,
                     w.nbias, t, T16, d.k_tiles * 256, perm, offsets, y, int(y_bf16));
  return hipGetLastError();
}

template <int SMAX, bool SPLIT>
hipError_t launch_s(const mbq_desc& d, const void* packed, int32_t t, const DecodeWs& w,
                    const int32_t* perm, const int32_t* offsets, void* y, bool y_bf16,
                    hipStream_t stream) {
  switch ((t + 15) / 16) {
    case 1: return launch_tb<1, SMAX, SPLIT>(d, packed, t, w, perm, offsets, y, y_bf16, stream);
    case 2: return launch_tb<2, SMAX, SPLIT>(d, packed, t, w, perm, offsets, y, y_bf16, stream);
    case 3: return launch_tb<3, SMAX, SPLIT>(d, packed, t, w, perm, offsets, y, y_bf16, stream);
    default: return launch_tb<4, SMAX, SPLIT>(d, packed, t, w, perm, offsets, y, y_bf16, stream);
  }
}

}  // namespace

size_t decode_workspace(const mbq_desc& d, int32_t t, bool x_bf16) {
  return carve(d, t, x_bf16, nullptr).bytes;
}

hipError_t launch_decode(const mbq_desc& d, const void* packed, int32_t t, const void* x,
                         bool x_bf16, const int32_t* perm, const int32_t* offsets, void* y,
                         bool y_bf16, void* ws, hipStream_t stream) {
  const DecodeWs w = carve(d, t, x_bf16, ws);
  const int T16 = ((t + 15) / 16) * 16;
  const int Kp = d.k_tiles * 256;
  const int total = T16 * (Kp / 16);
  dim3 pg((total + 255) / 256), pb(256);
  if (x_bf16)
    hipLaunchKernelGGL((xprep_kernel<true, false>), pg, pb, 0, stream, x, t, d.k, Kp, T16,
                       d.group, perm, w.xh, w.xl, w.xs, w.nbias);
  else
    hipLaunchKernelGGL((xprep_kernel<false, true>), pg, pb, 0, stream, x, t, d.k, Kp, T16,
                       d.group, perm, w.xh, w.xl, w.xs, w.nbias);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool split = !x_bf16;
  switch (d.slices) {
    case 1: return split ? launch_s<1, true>(d, packed, t, w, perm, offsets, y, y_bf16, stream)
                         : launch_s<1, false>(d, packed, t, w, perm, offsets, y, y_bf16, stream);
    case 2: return split ? launch_s<2, true>(d, packed, t, w, perm, offsets, y, y_bf16, stream)
                         : launch_s<2, false>(d, packed, t, w, perm, offsets, y, y_bf16, stream);
    case 3: return split ? launch_s<3, true>(d, packed, t, w, perm, offsets, y, y_bf16, stream)
                         : launch_s<3, false>(d, packed, t, w, perm, offsets, y, y_bf16, stream);
    default: return split ? launch_s<4, true>(d, packed, t, w, perm, offsets, y, y_bf16, stream)
                          : launch_s<4, false>(d, packed, t, w, perm, offsets, y, y_bf16, stream);
  }
}

}  // namespace mbq
