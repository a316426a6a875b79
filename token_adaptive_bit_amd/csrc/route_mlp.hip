// MoBiRoute in the form the pages give it: a 2-layer MLP scores every token once per
// residual slice, and at inference a sigmoid gate with threshold delta turns the scores
// into a binary mask; raising delta switches slices off (MoBiQuant explainer, gist.science,
// English section 2.B; the Japanese explainer, section 2.2).
//
//   hidden = ReLU(x . W1^T + b1)          W1 [H x K] bfloat16, b1 [H] float32
//   scores = hidden . W2 + b2             W2 [H x R] float32, b2 [R], R = S - 1
//   slice j + 1 passes when scores[j] > theta, theta = logit(delta) (sigmoid is
//   increasing, so this is the gate sigmoid(score) > delta without evaluating exp);
//   b(t) = 1 + the length of the leading run of passing slices, since each residual
//   slice refines the sum of the ones before it.
//
// Three steps on the device:
//   1. x . W1^T on bf16 MFMA (16x16x32, float32 accumulate), K split over workgroups so
//      the launch covers the chip.  Up to 64 tokens a workgroup owns 16 tokens x 64 units
//      and its four waves split the K chunk (summed through LDS); above that, 128 x 128
//      tiles are staged through LDS.  float32 activations enter the MFMA as a bf16
//      hi + lo pair (two products), which keeps about 16 mantissa bits.  Partial sums go
//      to the caller's workspace; no atomics, so results repeat exactly.
//   2. gate: one wave per token sums the K partials in a fixed order, adds b1, applies
//      the ReLU, takes the R dot products with W2 (fixed butterfly), adds b2 and applies
//      the threshold.  For t <= 64 one workgroup does all tokens and then the regroup.
//   3. for t > 64 the regroup is the stable counting sort shared with the linear router.
#include <type_traits>

#include "mbq_internal.h"

namespace mbq {
namespace {

constexpr int kHB = 64;         // hidden units per workgroup
constexpr int kU = 4;           // k steps (of 32 inputs) per load group
constexpr int kSmallT = 64;     // gate and regroup in one workgroup up to this many tokens
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past any resource: loads give 0

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;  // xor butterfly: every lane ends with the same bits
}

// Eight consecutive bf16 elements [k, k + 8) of one row, as an MFMA operand fragment.
// `off` is the byte offset of element k, or kOOB for a row outside the tensor.  VEC: K is
// a multiple of 8 and the row starts 16-byte aligned, so the eight are all in or all out.
template <bool VEC>
__device__ __forceinline__ u32x4_t load_bf16x8(__amdgpu_buffer_rsrc_t r, uint32_t off, int k, int K) {
  if (VEC) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, k < K ? off : kOOB, 0, 0));
  } else {
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      h[e] = __builtin_amdgcn_raw_buffer_load_b16(r, (k + e < K && off != kOOB) ? off + 2 * e : kOOB, 0, 0);
    return u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  }
}

// Eight float32 activations as raw bits (two 16-byte loads when VEC).
template <bool VEC>
__device__ __forceinline__ void load_f32x8(__amdgpu_buffer_rsrc_t r, uint32_t off, int k, int K,
                                           u32x4_t& lo4, u32x4_t& hi4) {
  if (VEC) {
    const uint32_t o = k < K ? off : kOOB;
    lo4 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
    hi4 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, o == kOOB ? kOOB : o + 16, 0, 0));
  } else {
    uint32_t f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      f[e] = __builtin_amdgcn_raw_buffer_load_b32(r, (k + e < K && off != kOOB) ? off + 4 * e : kOOB, 0, 0);
    lo4 = u32x4_t{f[0], f[1], f[2], f[3]};
    hi4 = u32x4_t{f[4], f[5], f[6], f[7]};
  }
}

// float32 x = hi + lo + O(2^-17 |x|): hi and lo are bf16, packed two per word.
__device__ __forceinline__ void split_f32x8(u32x4_t a, u32x4_t b, u32x4_t& hi, u32x4_t& lo) {
  const uint32_t f[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  uint32_t h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = bf16_bits_rne(__uint_as_float(f[e]));
    l[e] = bf16_bits_rne(__uint_as_float(f[e]) - bf16_bits_to_float(h[e]));
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    hi[w] = h[2 * w] | (h[2 * w + 1] << 16);
    lo[w] = l[2 * w] | (l[2 * w + 1] << 16);
  }
}

template <bool XBF16>
struct Frag {
  static constexpr int NA = XBF16 ? 1 : 2;  // raw activation words per fragment (x16 B)
  u32x4_t a[kU][NA];
  u32x4_t b[kU][4];
};

// t <= 64: partial hidden pre-activations of 16 tokens.  Grid: (token tiles of 16,
// H / 64, K chunks); 256 threads.  The four waves split the workgroup's K chunk, each
// holding the 16 x 64 product in MFMA accumulators, and LDS sums their parts.
// part[(chunk * T + t) * H + h] receives the chunk's sum for token t < T, hidden unit h.
template <bool XBF16, bool VEC>
__global__ __launch_bounds__(256) void mlp_hidden_small_kernel(const void* __restrict__ x, int T, int K,
                                                               const uint16_t* __restrict__ w1, int H,
                                                               int kpc, float* __restrict__ part,
                                                               int32_t* __restrict__ ready) {
  __shared__ float red[4][16][kHB];
  constexpr int ESZ = XBF16 ? 2 : 4;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // the gate's per-token budget words start at zero (gate_multi_kernel reads them in the
  // next launch)
  if ((blockIdx.x | blockIdx.y | blockIdx.z) == 0 && threadIdx.x < T) ready[threadIdx.x] = 0;
  const int h0 = blockIdx.y * kHB;
  const int t0 = blockIdx.x * 16;
  const int nsteps = (K + 31) >> 5;
  int sb = blockIdx.z * kpc, se = min(sb + kpc, nsteps);
  {
    const int q = (se - sb + 3) >> 2;
    sb = min(sb + wave * q, se);
    se = min(sb + q, se);
  }
  const __amdgpu_buffer_rsrc_t rx = rsrc(x, uint32_t(T) * uint32_t(K) * ESZ);
  const __amdgpu_buffer_rsrc_t rw = rsrc(w1, uint32_t(H) * uint32_t(K) * 2);
  const int row = t0 + (lane & 15), kq = 8 * (lane >> 4);
  // byte offsets of element kq of this lane's token row and of its four W1 rows
  const uint32_t xoff = row < T ? (uint32_t(row) * K + kq) * ESZ : kOOB;
  uint32_t woff[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) woff[n] = (uint32_t(h0 + 16 * n + (lane & 15)) * K + kq) * 2;

  auto load = [&](Frag<XBF16>& f, int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int s = s0 + u;
      const int k = (s < se) ? s * 32 + kq : K;  // steps past the range load zeros
      const uint32_t step = uint32_t(s) * 32 * ESZ;
      if (XBF16)
        f.a[u][0] = load_bf16x8<VEC>(rx, xoff == kOOB ? kOOB : xoff + step, k, K);
      else
        load_f32x8<VEC>(rx, xoff == kOOB ? kOOB : xoff + step, k, K, f.a[u][0], f.a[u][Frag<XBF16>::NA - 1]);
#pragma unroll
      for (int n = 0; n < 4; ++n) f.b[u][n] = load_bf16x8<VEC>(rw, woff[n] + uint32_t(s) * 64, k, K);
    }
  };

  f32x4_t acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Frag<XBF16>& f) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (XBF16) {
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[n] = mfma(f.a[u][0], f.b[u][n], acc[n]);
      } else {
        u32x4_t hi, lo;
        split_f32x8(f.a[u][0], f.a[u][Frag<XBF16>::NA - 1], hi, lo);
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[n] = mfma(hi, f.b[u][n], acc[n]);
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[n] = mfma(lo, f.b[u][n], acc[n]);
      }
    }
  };

  // Two load groups in flight: the next group is issued before this one is multiplied
  // (the two fragments alternate roles, so nothing is copied between them).  No branch
  // separates a load from its use inside the loop body, so the loads cannot be sunk
  // below the multiply they are meant to overlap; loads past the range return zeros and
  // touch no memory.
  const int ng = (se - sb + kU - 1) / kU;
  if (ng > 0) {
    Frag<XBF16> f0, f1;
    load(f0, sb);
    for (int g = 0; g + 2 <= ng; g += 2) {
      load(f1, sb + kU * (g + 1));
      compute(f0);
      load(f0, sb + kU * (g + 2));
      compute(f1);
    }
    if (ng & 1) compute(f0);
  }

  // lane holds hidden unit h0 + 16 n + lane % 16 for tokens t0 + 4 (lane / 16) + v
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int n = 0; n < 4; ++n) red[wave][4 * (lane >> 4) + v][16 * n + (lane & 15)] = acc[n][v];
  __syncthreads();
  const int r = threadIdx.x >> 4, c = 4 * (threadIdx.x & 15);
  const int t = t0 + r;
  if (t < T) {
    float4 o;
    o.x = ((red[0][r][c + 0] + red[1][r][c + 0]) + red[2][r][c + 0]) + red[3][r][c + 0];
    o.y = ((red[0][r][c + 1] + red[1][r][c + 1]) + red[2][r][c + 1]) + red[3][r][c + 1];
    o.z = ((red[0][r][c + 2] + red[1][r][c + 2]) + red[2][r][c + 2]) + red[3][r][c + 2];
    o.w = ((red[0][r][c + 3] + red[1][r][c + 3]) + red[2][r][c + 3]) + red[3][r][c + 3];
    *reinterpret_cast<float4*>(part + (size_t(blockIdx.z) * T + t) * H + h0 + c) = o;
  }
}

// t > 64: 128-token x 128-unit output tiles with both operands staged through LDS.
// Every row segment a workgroup loads is 128 contiguous bytes (64 bf16 inputs; float32
// x rows are 256), so each cache line is fetched whole and once per tile, and the four
// waves (a 2 x 2 grid of 64 x 64 sub-tiles, 16 MFMAs per 32 inputs each) share both
// operands from LDS.  Grid: (token tiles, unit tiles, K chunks of kpc 64-input stages).
constexpr int kBM = 128, kBN = 128, kBK = 64, kLDK = kBK + 8;  // LDS row: 64 inputs + 16 B pad

template <bool XBF16, bool VEC>
__global__ __launch_bounds__(256) void mlp_hidden_tiled_kernel(const void* __restrict__ x, int T, int K,
                                                               const uint16_t* __restrict__ w1, int H,
                                                               int kpc, float* __restrict__ part) {
  constexpr int NA = XBF16 ? 1 : 2;  // A planes: bf16 x, or the hi and lo halves of float32 x
  constexpr int ESZ = XBF16 ? 2 : 4;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][NA][kBM * kLDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBN * kLDK];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int t0 = blockIdx.x * kBM, h0 = blockIdx.y * kBN;
  const int nst = (K + kBK - 1) / kBK;
  const int sb = blockIdx.z * kpc, se = min(sb + kpc, nst);
  const __amdgpu_buffer_rsrc_t rx = rsrc(x, uint32_t(T) * uint32_t(K) * ESZ);
  const __amdgpu_buffer_rsrc_t rw = rsrc(w1, uint32_t(H) * uint32_t(K) * 2);

  // staging: thread -> rows srow + 32 i (i < 4) of both tiles, inputs skc .. skc + 7
  const int srow = tid >> 3, skc = 8 * (tid & 7);
  uint32_t xo[4], wo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = srow + 32 * i;
    xo[i] = t0 + r < T ? (uint32_t(t0 + r) * K + skc) * ESZ : kOOB;
    wo[i] = h0 + r < H ? (uint32_t(h0 + r) * K + skc) * 2 : kOOB;
  }
  struct Stage {
    u32x4_t a[4][NA];
    u32x4_t b[4];
  };
  auto gload = [&](Stage& g, int st) __attribute__((always_inline)) {
    const int k = st < se ? st * kBK + skc : K;  // stages past the chunk load zeros
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t xs = xo[i] == kOOB ? kOOB : xo[i] + uint32_t(st) * (kBK * ESZ);
      if (XBF16)
        g.a[i][0] = load_bf16x8<VEC>(rx, xs, k, K);
      else
        load_f32x8<VEC>(rx, xs, k, K, g.a[i][0], g.a[i][NA - 1]);
      g.b[i] = load_bf16x8<VEC>(rw, wo[i] == kOOB ? kOOB : wo[i] + uint32_t(st) * (kBK * 2), k, K);
    }
  };
  auto swrite = [&](const Stage& g, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = (srow + 32 * i) * kLDK + skc;
      if (XBF16) {
        *reinterpret_cast<u32x4_t*>(&As[buf][0][o]) = g.a[i][0];
      } else {
        u32x4_t hi, lo;
        split_f32x8(g.a[i][0], g.a[i][NA - 1], hi, lo);
        *reinterpret_cast<u32x4_t*>(&As[buf][0][o]) = hi;
        *reinterpret_cast<u32x4_t*>(&As[buf][NA - 1][o]) = lo;
      }
      *reinterpret_cast<u32x4_t*>(&Bs[buf][o]) = g.b[i];
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      const int fo = (lane & 15) * kLDK + kk + 8 * (lane >> 4);
      u32x4_t a[4][NA], b[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int p = 0; p < NA; ++p)
          a[mi][p] = *reinterpret_cast<const u32x4_t*>(&As[buf][p][(64 * wm + 16 * mi) * kLDK + fo]);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        b[ni] = *reinterpret_cast<const u32x4_t*>(&Bs[buf][(64 * wn + 16 * ni) * kLDK + fo]);
#pragma unroll
      for (int p = 0; p < NA; ++p)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma(a[mi][p], b[ni], acc[mi][ni]);
    }
  };

  // One barrier per stage.  Two stages are in flight from memory while one is multiplied:
  // stage st + 2 is requested before stage st is multiplied, and stage st + 1 (requested
  // a stage earlier) is then written into the other LDS buffer, whose last readers (stage
  // st - 1) finished before the previous barrier.  The loop runs in pairs of stages so the
  // two register stages never trade places; an odd count multiplies one stage of zeros.
  if (sb < se) {
    Stage g0, g1;
    gload(g0, sb);
    gload(g1, sb + 1);
    swrite(g0, 0);
    __syncthreads();
    for (int st = sb; st < se; st += 2) {
      gload(g0, st + 2);
      compute(0);
      swrite(g1, 1);
      __syncthreads();
      gload(g1, st + 3);
      compute(1);
      swrite(g0, 0);
      __syncthreads();
    }
  }

  // lane holds unit h0 + 64 wn + 16 ni + lane % 16 of tokens t0 + 64 wm + 16 mi + 4 (lane / 16) + v
  float* dst = part + size_t(blockIdx.z) * T * H;
  const int hb = h0 + 64 * wn + (lane & 15);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = t0 + 64 * wm + 16 * mi + 4 * (lane >> 4) + v;
      if (t < T)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          if (hb + 16 * ni < H) dst[size_t(t) * H + hb + 16 * ni] = acc[mi][ni][v];
    }
}

// Scores and budget of token t, computed by one wave; the result is wave-uniform.
// SCORES_IN: the scores are read from `scores` instead of computed.
template <int R, bool SCORES_IN>
__device__ __forceinline__ int token_budget(int t, int T, int H, int KS, const float* __restrict__ part,
                                            const float* __restrict__ b1, const float* __restrict__ w2,
                                            const float* __restrict__ b2, float theta,
                                            float* __restrict__ scores, int lane) {
  if (R == 0) return 1;
  float sc[R > 0 ? R : 1];
  if (SCORES_IN) {
#pragma unroll
    for (int r = 0; r < R; ++r) sc[r] = scores[size_t(t) * R + r];
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) sc[r] = 0.f;
    for (int h = 4 * lane; h < H; h += 256) {
      // Chunk partials summed in chunk order.  Sixteen loads are issued before the first
      // add; past the last chunk the index is clamped and the term weighted by 0, which
      // leaves the sum unchanged (a + 1 * p rounds like a + p; a + 0 * p is a).
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int k0 = 0; k0 < KS; k0 += 16) {
        float4 p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          p[i] = *reinterpret_cast<const float4*>(part + (size_t(min(k0 + i, KS - 1)) * T + t) * H + h);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float m = k0 + i < KS ? 1.f : 0.f;
          a.x = fmaf(p[i].x, m, a.x); a.y = fmaf(p[i].y, m, a.y);
          a.z = fmaf(p[i].z, m, a.z); a.w = fmaf(p[i].w, m, a.w);
        }
      }
      const float4 bb = *reinterpret_cast<const float4*>(b1 + h);
      const float hv[4] = {fmaxf(a.x + bb.x, 0.f), fmaxf(a.y + bb.y, 0.f), fmaxf(a.z + bb.z, 0.f),
                           fmaxf(a.w + bb.w, 0.f)};
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int r = 0; r < R; ++r) sc[r] = fmaf(hv[e], w2[size_t(h + e) * R + r], sc[r]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) sc[r] = wave_sum(sc[r]) + b2[r];
    if (lane == 0)
#pragma unroll
      for (int r = 0; r < R; ++r) scores[size_t(t) * R + r] = sc[r];
  }
  int b = 1;
  bool run = true;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    run = run && (sc[r] > theta);
    b += run ? 1 : 0;
  }
  return b;
}

// t > 64: one wave per token; the regroup follows as a separate launch.
template <int R, bool SCORES_IN>
__global__ __launch_bounds__(256) void gate_kernel(int T, int H, int KS, const float* __restrict__ part,
                                                   const float* __restrict__ b1, const float* __restrict__ w2,
                                                   const float* __restrict__ b2, float theta,
                                                   float* __restrict__ scores, int32_t* __restrict__ budget) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform
  const int b = token_budget<R, SCORES_IN>(t, T, H, KS, part, b1, w2, b2, theta, scores, lane);
  if (lane == 0) budget[t] = b;
}

// t <= 64 with the hidden layer computed in the launch before: one wave per token over
// ceil(t / 4) workgroups, so the chunk partials are read by several CUs at once.  Each wave
// publishes its token's budget (>= 1) in a word the hidden launch cleared; wave 0 of
// workgroup 0 then waits until every word is set and regroups with ballot ranks, as
// gate_small_kernel does.  A budget is one word, so seeing it non-zero is seeing it whole.
// The wait is bounded (a workgroup that never ran would leave its tokens at budget 1).
constexpr int kGateSpin = 1 << 16;

template <int R>
__global__ __launch_bounds__(256) void gate_multi_kernel(int T, int S, int H, int KS,
                                                         const float* __restrict__ part,
                                                         const float* __restrict__ b1,
                                                         const float* __restrict__ w2,
                                                         const float* __restrict__ b2, float theta,
                                                         float* __restrict__ scores, int32_t* __restrict__ budget,
                                                         int32_t* __restrict__ perm, int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ ready) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;  // wave-uniform
  const int bt = token_budget<R, false>(t, T, H, KS, part, b1, w2, b2, theta, scores, lane);
  if (lane == 0) __hip_atomic_store(ready + t, bt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (blockIdx.x != 0 || wave != 0) return;
  int bl = 1;
  for (int it = 0;; ++it) {
    bl = lane < T ? __hip_atomic_load(ready + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 1;
    if (__ballot(bl == 0) == 0ull) break;
    if (it >= kGateSpin) {
      bl = bl == 0 ? 1 : bl;
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  const int b = lane < T ? bl : 0;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int base = 0, pos = 0;
  if (lane == 0) offsets[0] = 0;
  for (int v = 1; v <= S; ++v) {
    const uint64_t m = __ballot(b == v);
    if (b == v) pos = base + __popcll(m & lt);
    base += __popcll(m);
    if (lane == 0) offsets[v] = base;
  }
  if (lane < T) {
    perm[pos] = lane;
    budget[lane] = b;
  }
}

// t <= 64 with the scores given: sixteen waves gate the tokens, then wave 0 regroups them
// with ballot ranks (stable: ranks follow token order within each budget).
template <int R, bool SCORES_IN>
__global__ __launch_bounds__(1024) void gate_small_kernel(int T, int S, int H, int KS,
                                                          const float* __restrict__ part,
                                                          const float* __restrict__ b1,
                                                          const float* __restrict__ w2,
                                                          const float* __restrict__ b2, float theta,
                                                          float* __restrict__ scores,
                                                          int32_t* __restrict__ budget,
                                                          int32_t* __restrict__ perm,
                                                          int32_t* __restrict__ offsets) {
  __shared__ int bs[kSmallT];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int t = wave; t < T; t += 16) {
    const int b = token_budget<R, SCORES_IN>(t, T, H, KS, part, b1, w2, b2, theta, scores, lane);
    if (lane == 0) bs[t] = b;
  }
  __syncthreads();
  if (wave != 0) return;
  const int b = lane < T ? bs[lane] : 0;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int base = 0, pos = 0;
  if (lane == 0) offsets[0] = 0;
  for (int v = 1; v <= S; ++v) {
    const uint64_t m = __ballot(b == v);
    if (b == v) pos = base + __popcll(m & lt);
    base += __popcll(m);
    if (lane == 0) offsets[v] = base;
  }
  if (lane < T) {
    perm[pos] = lane;
    budget[lane] = b;
  }
}

struct MlpPlan {
  bool tiled;
  int tiles, hblocks, ks, kpc;
};

MlpPlan mlp_plan(int32_t t, int32_t k, int32_t h) {
  MlpPlan p;
  p.tiled = t > kSmallT;
  int nst, base, ks;
  if (!p.tiled) {  // 16-token tiles, 64 units, 32-input steps, >= 2 steps per wave
    p.tiles = (t + 15) / 16;
    p.hblocks = h / kHB;
    nst = (k + 31) / 32;
    base = p.tiles * p.hblocks;
    ks = std::min((256 + base - 1) / base, std::max(1, nst / 8));
  } else {         // 128 x 128 tiles, 64-input stages, >= 2 stages per chunk, <= 16 chunks
    p.tiles = (t + kBM - 1) / kBM;
    p.hblocks = (h + kBN - 1) / kBN;
    nst = (k + kBK - 1) / kBK;
    base = p.tiles * p.hblocks;
    ks = std::min(std::min((256 + base - 1) / base, 16), std::max(1, nst / 2));
  }
  ks = std::max(1, std::min(ks, 64));
  p.kpc = (nst + ks - 1) / ks;
  p.ks = (nst + p.kpc - 1) / p.kpc;
  return p;
}

}  // namespace

// chunk partials [ks x t x h] float32, then (t <= 64) 256 bytes of per-token budget words
size_t route_mlp_workspace(int32_t t, int32_t k, int32_t h) {
  if (t <= 0) return 0;
  const MlpPlan p = mlp_plan(t, k, h);
  return size_t(p.ks) * size_t(t) * size_t(h) * sizeof(float) + (t <= kSmallT ? 256 : 0);
}

hipError_t launch_route_mlp(int32_t t, int32_t k, int32_t s, int32_t h, const void* x, bool x_bf16,
                            const uint16_t* w1, const float* b1, const float* w2, const float* b2,
                            float theta, float* scores, int32_t* budget, int32_t* perm,
                            int32_t* offsets, void* ws, hipStream_t stream) {
  const int R = s - 1;
  const bool scores_in = x == nullptr;
  MlpPlan p{false, 0, 0, 1, 0};
  if (t > 0 && R > 0 && !scores_in) {
    p = mlp_plan(t, k, h);
    const bool vec = k % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(w1) & 15) == 0;
    const dim3 grid(p.tiles, p.hblocks, p.ks);
    float* part = static_cast<float*>(ws);
    int32_t* ready = reinterpret_cast<int32_t*>(part + size_t(p.ks) * size_t(t) * size_t(h));
    auto go = [&](auto xb, auto vv) {
      constexpr bool XB = decltype(xb)::value, VV = decltype(vv)::value;
      if (p.tiled)
        hipLaunchKernelGGL((mlp_hidden_tiled_kernel<XB, VV>), grid, dim3(256), 0, stream, x, t, k, w1,
                           h, p.kpc, part);
      else
        hipLaunchKernelGGL((mlp_hidden_small_kernel<XB, VV>), grid, dim3(256), 0, stream, x, t, k, w1,
                           h, p.kpc, part, ready);
    };
    auto go_v = [&](auto xb) {
      if (vec) go(xb, std::true_type{});
      else go(xb, std::false_type{});
    };
    if (x_bf16) go_v(std::true_type{});
    else go_v(std::false_type{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const float* part = static_cast<const float*>(ws);
  auto gate = [&](auto rr, auto si) {
    constexpr int RR = decltype(rr)::value;
    constexpr bool SI = decltype(si)::value;
    if (t <= kSmallT && !SI && RR > 0)  // (the hidden launch ran and cleared the budget words)
      hipLaunchKernelGGL((gate_multi_kernel<RR>), dim3((t + 3) / 4), dim3(256), 0, stream, t, s, h, p.ks,
                         part, b1, w2, b2, theta, scores, budget, perm, offsets,
                         const_cast<int32_t*>(reinterpret_cast<const int32_t*>(part + size_t(p.ks) * size_t(t) * size_t(h))));
    else if (t <= kSmallT)
      hipLaunchKernelGGL((gate_small_kernel<RR, SI>), dim3(1), dim3(1024), 0, stream, t, s, h, p.ks,
                         part, b1, w2, b2, theta, scores, budget, perm, offsets);
    else
      hipLaunchKernelGGL((gate_kernel<RR, SI>), dim3((t + 3) / 4), dim3(256), 0, stream, t, h, p.ks,
                         part, b1, w2, b2, theta, scores, budget);
  };
  auto gate_r = [&](auto si) {
    switch (R) {
      case 0: gate(std::integral_constant<int, 0>{}, si); break;
      case 1: gate(std::integral_constant<int, 1>{}, si); break;
      case 2: gate(std::integral_constant<int, 2>{}, si); break;
      default: gate(std::integral_constant<int, 3>{}, si); break;
    }
  };
  if (scores_in) gate_r(std::true_type{});
  else gate_r(std::false_type{});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || t <= kSmallT) return e;
  return launch_route(t, 0, s, nullptr, false, nullptr, nullptr, budget, nullptr, perm, offsets,
                      stream);
}

}  // namespace mbq
