// Low-rank side path of a quantized linear: W ~ Wq + B A, so y_t = x_t . Wq^T + u_t . B^T
// with u_t = x_t . A^T (TTQ explainer, gist.science, Japanese, section 2: the quantized
// weight plus rank-r factors kept beside it; section 4: rank 16 costs little).  Here Wq is
// the token's MoBiSlice sum W^(b(t)), and one (A, B) pair serves every token.
//
// This file computes u (float32, [T x R], original token order) for the routed linear
// kernels, which add u_t . B^T to their accumulators before storing (streaming decode:
// two MFMAs per row block; MFMA prefill: two per output block after the last chunk).  The
// generic fallback kernels add it afterwards with lowrank_update_kernel.
//
// lowrank_u_kernel: workgroups of 4 waves over 16 tokens x one of KSU chunks of K (few
// tokens get several chunks, so the launch spreads over the chip).  The waves split the
// chunk into contiguous ranges of 32-input steps; each multiplies 16 tokens x 16 ranks per
// step on bf16 MFMA (float32 x as a bf16 hi + lo pair) with two load groups in flight,
// and LDS sums the 4 partial tiles in a fixed order.  (16 waves per workgroup, each with
// fewer steps, measured 0.5 us slower per decode step at 16 tokens, K = 3584.)  Chunk z writes u_part[z] [T x R];
// the consumers add the chunks in order 0, 1, ..., so u repeats exactly from run to run.
#include <type_traits>

#include "mbq_internal.h"

namespace mbq {
namespace {

constexpr int kU = 4;                   // 32-input steps per load group
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past any resource: loads give 0

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

// Eight bf16 elements [k, k + 8) at byte offset off (kOOB: zeros).  VEC: 16-byte loads
// (K % 8 == 0 and aligned rows); otherwise element loads.
template <bool VEC>
__device__ __forceinline__ u32x4_t ld_bf16x8(__amdgpu_buffer_rsrc_t r, uint32_t off, int k, int K) {
  if (VEC)
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, k < K ? off : kOOB, 0, 0));
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    h[e] = __builtin_amdgcn_raw_buffer_load_b16(r, (k + e < K && off != kOOB) ? off + 2 * e : kOOB, 0, 0);
  return u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

template <bool VEC>
__device__ __forceinline__ void ld_f32x8(__amdgpu_buffer_rsrc_t r, uint32_t off, int k, int K,
                                         u32x4_t& a, u32x4_t& b) {
  if (VEC) {
    const uint32_t o = k < K ? off : kOOB;
    a = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
    b = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, o == kOOB ? kOOB : o + 16, 0, 0));
    return;
  }
  uint32_t f[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    f[e] = __builtin_amdgcn_raw_buffer_load_b32(r, (k + e < K && off != kOOB) ? off + 4 * e : kOOB, 0, 0);
  a = u32x4_t{f[0], f[1], f[2], f[3]};
  b = u32x4_t{f[4], f[5], f[6], f[7]};
}

// float32 x = hi + lo + O(2^-17 |x|), hi and lo bf16, two per word.
__device__ __forceinline__ void split8(u32x4_t a, u32x4_t b, u32x4_t& hi, u32x4_t& lo) {
  const uint32_t f[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t h[2], l[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float v = __uint_as_float(f[2 * w + e]);
      h[e] = bf16_bits_rne(v);
      l[e] = bf16_bits_rne(v - bf16_bits_to_float(h[e]));
    }
    hi[w] = h[0] | (h[1] << 16);
    lo[w] = l[0] | (l[1] << 16);
  }
}

template <bool XBF16, int NF>
struct LrFrag {
  static constexpr int NA = XBF16 ? 1 : 2;
  u32x4_t a[kU][NA];
  u32x4_t b[kU][NF];
};

// u_part [KSU x T x R]: chunk blockIdx.y of x [T x K] . A^T, A [R x K] bf16.
// NF = ceil(R / 16) rank fragments; kpc 32-input steps per chunk.
constexpr int kUWaves = 4;

template <bool XBF16, bool VEC, int NF>
__global__ __launch_bounds__(64 * kUWaves) void lowrank_u_kernel(const void* __restrict__ x, int T, int K,
                                                                 const uint16_t* __restrict__ A, int R,
                                                                 int kpc, float* __restrict__ u) {
  constexpr int NW = kUWaves, ESZ = XBF16 ? 2 : 4;
  __shared__ float red[NW][16][16 * NF];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * 16;
  const int nsteps = (K + 31) >> 5;
  const int cb = min(int(blockIdx.y) * kpc, nsteps), ce = min(cb + kpc, nsteps);
  const int q = (ce - cb + NW - 1) / NW;
  const int sb = min(cb + wave * q, ce), se = min(sb + q, ce);
  const __amdgpu_buffer_rsrc_t rx = rsrc(x, uint32_t(T) * uint32_t(K) * ESZ);
  const __amdgpu_buffer_rsrc_t ra = rsrc(A, uint32_t(R) * uint32_t(K) * 2);
  const int row = t0 + (lane & 15), kq = 8 * (lane >> 4);
  const uint32_t xoff = row < T ? (uint32_t(row) * K + kq) * ESZ : kOOB;
  uint32_t aoff[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int ar = 16 * f + (lane & 15);
    aoff[f] = ar < R ? (uint32_t(ar) * K + kq) * 2 : kOOB;
  }
  auto load = [&](LrFrag<XBF16, NF>& g, int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int uu = 0; uu < kU; ++uu) {
      const int s = s0 + uu;
      const int k = s < se ? s * 32 + kq : K;  // steps past the range load zeros
      const uint32_t xs = xoff == kOOB ? kOOB : xoff + uint32_t(s) * 32 * ESZ;
      if (XBF16)
        g.a[uu][0] = ld_bf16x8<VEC>(rx, xs, k, K);
      else
        ld_f32x8<VEC>(rx, xs, k, K, g.a[uu][0], g.a[uu][LrFrag<XBF16, NF>::NA - 1]);
#pragma unroll
      for (int f = 0; f < NF; ++f)
        g.b[uu][f] = ld_bf16x8<VEC>(ra, aoff[f] == kOOB ? kOOB : aoff[f] + uint32_t(s) * 64, k, K);
    }
  };
  f32x4_t acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const LrFrag<XBF16, NF>& g) __attribute__((always_inline)) {
#pragma unroll
    for (int uu = 0; uu < kU; ++uu) {
      if (XBF16) {
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[f] = mfma(g.a[uu][0], g.b[uu][f], acc[f]);
      } else {
        u32x4_t hi, lo;
        split8(g.a[uu][0], g.a[uu][LrFrag<XBF16, NF>::NA - 1], hi, lo);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          acc[f] = mfma(hi, g.b[uu][f], acc[f]);
          acc[f] = mfma(lo, g.b[uu][f], acc[f]);
        }
      }
    }
  };
  // two load groups in flight; no branch between a load and its use (see route_mlp.hip)
  const int ng = (se - sb + kU - 1) / kU;
  if (ng > 0) {
    LrFrag<XBF16, NF> f0, f1;
    load(f0, sb);
    for (int g = 0; g + 2 <= ng; g += 2) {
      load(f1, sb + kU * (g + 1));
      compute(f0);
      load(f0, sb + kU * (g + 2));
      compute(f1);
    }
    if (ng & 1) compute(f0);
  }
  // lane holds rank 16 f + lane % 16 of tokens t0 + 4 (lane / 16) + v
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][4 * (lane >> 4) + v][16 * f + (lane & 15)] = acc[f][v];
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * 16 * NF; i += blockDim.x) {
    const int tr = i / (16 * NF), rr = i % (16 * NF);
    if (t0 + tr < T && rr < R) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += red[w][tr][rr];
      u[(size_t(blockIdx.y) * T + t0 + tr) * R + rr] = s;
    }
  }
}

// y[t][n] += sum_r u[t][r] B[n][r] (float32 accumulate, fixed order), for the generic
// kernels; u[t][r] is the sum of the KSU chunks in order.  One thread per (t, n); y is
// float32 or bfloat16 (rounded again).
__global__ __launch_bounds__(256) void lowrank_update_kernel(const float* __restrict__ u, int ksu,
                                                             const uint16_t* __restrict__ B, int T, int N,
                                                             int R, void* __restrict__ y, int y_bf16) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  for (int t = blockIdx.y; t < T; t += gridDim.y) {
    float s = 0.f;
    for (int r = 0; r < R; ++r) {
      float ur = u[size_t(t) * R + r];
      for (int z = 1; z < ksu; ++z) ur += u[(size_t(z) * T + t) * R + r];
      s = fmaf(ur, bf16_bits_to_float(B[size_t(n) * R + r]), s);
    }
    const size_t i = size_t(t) * N + n;
    if (y_bf16) {
      uint16_t* p = static_cast<uint16_t*>(y) + i;
      *p = uint16_t(bf16_bits_rne(bf16_bits_to_float(*p) + s));
    } else {
      float* p = static_cast<float*>(y) + i;
      *p = *p + s;
    }
  }
}

}  // namespace

int lowrank_u_chunks(int32_t t, int32_t k) {
  if (t <= 0) return 1;
  const int tiles = (t + 15) / 16, nsteps = (k + 31) / 32;
  // about 128 workgroups, every wave with at least one 32-input step, at most 8 chunks
  const int ksu = std::min(std::min((128 + tiles - 1) / tiles, kMaxLrChunks), std::max(1, nsteps / 16));
  const int kpc = (nsteps + ksu - 1) / ksu;
  return (nsteps + kpc - 1) / kpc;
}

hipError_t launch_lowrank_u(int32_t t, int32_t k, const void* x, bool x_bf16, const uint16_t* a,
                            int32_t rank, float* u, hipStream_t stream) {
  if (t <= 0) return hipSuccess;
  const bool vec = k % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(a) & 15) == 0;
  const int nsteps = (k + 31) / 32, ksu = lowrank_u_chunks(t, k);
  const int kpc = (nsteps + ksu - 1) / ksu;
  const dim3 grid((t + 15) / 16, ksu);
  auto go = [&](auto xb, auto vv, auto nf) {
    hipLaunchKernelGGL((lowrank_u_kernel<decltype(xb)::value, decltype(vv)::value, decltype(nf)::value>),
                       grid, dim3(64 * kUWaves), 0, stream, x, t, k, a, rank, kpc, u);
  };
  auto go_nf = [&](auto xb, auto vv) {
    if (rank > 16) go(xb, vv, std::integral_constant<int, 2>{});
    else go(xb, vv, std::integral_constant<int, 1>{});
  };
  auto go_v = [&](auto xb) {
    if (vec) go_nf(xb, std::true_type{});
    else go_nf(xb, std::false_type{});
  };
  if (x_bf16) go_v(std::true_type{});
  else go_v(std::false_type{});
  return hipGetLastError();
}

hipError_t launch_lowrank_update(int32_t t, int32_t n, const float* u, int32_t ksu, const uint16_t* b,
                                 int32_t rank, void* y, bool y_bf16, hipStream_t stream) {
  if (t <= 0) return hipSuccess;
  hipLaunchKernelGGL(lowrank_update_kernel, dim3((n + 255) / 256, std::min(t, 4096)), dim3(256), 0,
                     stream, u, ksu, b, t, n, rank, y, int(y_bf16));
  return hipGetLastError();
}

}  // namespace mbq
