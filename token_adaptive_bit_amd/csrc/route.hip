// MoBiRoute, linear-argmax form, and the token regroup.
//
// MoBiQuant explainer (gist.science, English), section 2.B: a lightweight router scores
// each token and the scores decide how many residual slices the token activates.  Here
// the score is logits = x . Wr (float32 accumulate) and b(t) = 1 + the first index of the
// largest logit.  Tokens are then regrouped by a stable ascending sort on b(t) so that
// the linear kernels see runs of tokens with one budget (the pages leave the regroup
// open; the English page, section 5, names irregular access as the cost it avoids).
//
// The logits kernel runs one workgroup per token (coalesced loads, fixed-order sums, so
// logits and routes are identical from run to run).  The sort runs in one wave with
// ballot ranks for T <= 64 (decode) and in one 1024-thread workgroup otherwise.
#include <type_traits>

#include "mbq_internal.h"

namespace mbq {
namespace {

constexpr int kSmallT = 64;

// sum over the wave, fixed butterfly order
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Partial dot products of one token row against Wr: thread i takes inputs i, i + stride,
// ...; consecutive threads read consecutive activations and consecutive Wr rows, so every
// load instruction is coalesced.
template <bool BF16>
__device__ __forceinline__ void dot_row(const void* __restrict__ x, size_t row, int K, int S,
                                        const float* __restrict__ wr, int i0, int stride,
                                        float (&acc)[4]) {
  constexpr int U = 8;  // independent loads in flight per thread
  for (int k0 = i0; k0 < K; k0 += U * stride) {
    float xk[U], w[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + u * stride;
      const bool in = k < K;
      xk[u] = in ? load_x(x, row * K + k, BF16) : 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) w[u][s] = (in && s < S) ? wr[size_t(k) * S + s] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[s] = fmaf(xk[u], w[u][s], acc[s]);
  }
}

__device__ __forceinline__ int argmax_first(const float* l, int S) {
  float best = l[0];
  int arg = 0;
  for (int j = 1; j < S; ++j)
    if (l[j] > best) { best = l[j]; arg = j; }
  return arg + 1;
}

// T <= 64: budgets, perm and offsets from the logits in one wave (ballot ranks).
__global__ __launch_bounds__(64) void route_small_kernel(int T, int S, const float* __restrict__ logits,
                                                         int32_t* __restrict__ budget,
                                                         int32_t* __restrict__ perm,
                                                         int32_t* __restrict__ offsets) {
  const int lane = threadIdx.x;
  const int b = lane < T ? argmax_first(logits + size_t(lane) * S, S) : 0;
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

// One workgroup (512 threads) per token.  With 16-byte aligned x and Wr and K % 8 == 0,
// thread i takes 8-input chunks i, i + 512, ...: one 16-byte activation load (two for
// float32) and 2 S 16-byte Wr loads per chunk, every chunk's loads in flight at once up
// to kVecChunks; otherwise the scalar strided loop.
constexpr int kVecChunks = 4;

template <bool BF16, int S>
__device__ __forceinline__ void dot_row_vec(const void* __restrict__ x, size_t row, int K,
                                            const float* __restrict__ wr, int i0,
                                            float (&acc)[4]) {
  constexpr int XV = BF16 ? 1 : 2;
  const int K8 = K >> 3;
  for (int cb = i0; cb < K8; cb += 512 * kVecChunks) {
    u32x4_t xr[kVecChunks][XV];
    f32x4_t wv[kVecChunks][2 * S];
#pragma unroll
    for (int u = 0; u < kVecChunks; ++u) {
      const int ch = cb + 512 * u;
      if (ch < K8) {
        const uint8_t* px = static_cast<const uint8_t*>(x) + (row * K + size_t(ch) * 8) * (BF16 ? 2 : 4);
#pragma unroll
        for (int q = 0; q < XV; ++q) xr[u][q] = *reinterpret_cast<const u32x4_t*>(px + 16 * q);
#pragma unroll
        for (int v = 0; v < 2 * S; ++v)
          wv[u][v] = reinterpret_cast<const f32x4_t*>(wr + size_t(ch) * 8 * S)[v];
      }
    }
#pragma unroll
    for (int u = 0; u < kVecChunks; ++u) {
      if (cb + 512 * u >= K8) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xe = BF16 ? __uint_as_float((e & 1) ? (xr[u][0][e >> 1] & 0xFFFF0000u)
                                                         : (xr[u][0][e >> 1] << 16))
                              : __uint_as_float(xr[u][e >> 2][e & 3]);
#pragma unroll
        for (int q = 0; q < S; ++q) acc[q] = fmaf(xe, wv[u][(e * S + q) >> 2][(e * S + q) & 3], acc[q]);
      }
    }
  }
}

template <bool BF16, int SV>
__global__ __launch_bounds__(512) void logits_kernel(const void* __restrict__ x, int T, int K,
                                                     int S, const float* __restrict__ wr,
                                                     float* __restrict__ logits) {
  __shared__ float part[8][4];
  const int t = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (SV > 0)
    dot_row_vec<BF16, (SV > 0 ? SV : 1)>(x, size_t(t), K, wr, threadIdx.x, acc);
  else
    dot_row<BF16>(x, size_t(t), K, S, wr, threadIdx.x, 512, acc);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const float v = wave_sum(acc[s]);
    if (lane == 0) part[wave][s] = v;
  }
  __syncthreads();
  if (threadIdx.x < S) {
    const int s = threadIdx.x;
    logits[size_t(t) * S + s] = ((part[0][s] + part[1][s]) + (part[2][s] + part[3][s])) +
                                ((part[4][s] + part[5][s]) + (part[6][s] + part[7][s]));
  }
}

// One workgroup of 1024 threads: histogram of budgets, then a stable scatter in token
// order, 1024 tokens per step, using wave ballots for the in-wave rank.
__global__ __launch_bounds__(1024) void route_kernel(int T, int S, const float* __restrict__ logits,
                                                     const int32_t* __restrict__ budget_in,
                                                     int32_t* __restrict__ budget_out,
                                                     int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ offsets) {
  __shared__ int cnt[5];
  __shared__ int wave_tot[16][5];
  __shared__ int running[5];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  auto budget_of = [&](int t) -> int {
    if (budget_in) {
      int b = budget_in[t];
      return b < 1 ? 1 : (b > S ? S : b);  // out-of-contract values are clamped, never used as addresses
    }
    return argmax_first(logits + size_t(t) * S, S);
  };

  if (tid < 5) cnt[tid] = 0;
  __syncthreads();
  for (int t = tid; t < T; t += 1024) atomicAdd(&cnt[budget_of(t)], 1);
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    offsets[0] = 0;
    running[0] = 0;
    for (int v = 1; v <= S; ++v) {
      running[v] = acc;  // first sorted position of budget v
      acc += cnt[v];
      offsets[v] = acc;
    }
  }
  __syncthreads();
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < T; base += 1024) {
    const int t = base + tid;
    const int b = (t < T) ? budget_of(t) : 0;
    int rank = 0;
    for (int v = 1; v <= S; ++v) {
      const uint64_t m = __ballot(b == v);
      if (b == v) rank = __popcll(m & lt);
      if (lane == 0) wave_tot[wave][v] = __popcll(m);
    }
    __syncthreads();
    if (t < T) {
      int pre = running[b];
      for (int w = 0; w < wave; ++w) pre += wave_tot[w][b];
      perm[pre + rank] = t;
      if (budget_out) budget_out[t] = b;
    }
    __syncthreads();
    if (tid == 0)
      for (int v = 1; v <= S; ++v) {
        int tot = 0;
        for (int w = 0; w < 16; ++w) tot += wave_tot[w][v];
        running[v] += tot;
      }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_route(int32_t t, int32_t k, int32_t s, const void* x, bool x_bf16,
                        const float* wr, float* logits, const int32_t* budget_in,
                        int32_t* budget, int32_t* perm, int32_t* offsets, hipStream_t stream) {
  if (x && t > 0) {
    const bool vec = k % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(wr) & 15) == 0;
    auto go = [&](auto bf, auto sv) {
      hipLaunchKernelGGL((logits_kernel<decltype(bf)::value, decltype(sv)::value>), dim3(t),
                         dim3(512), 0, stream, x, t, k, s, wr, logits);
    };
    auto go_s = [&](auto bf) {
      switch (vec ? s : 0) {
        case 1: go(bf, std::integral_constant<int, 1>{}); break;
        case 2: go(bf, std::integral_constant<int, 2>{}); break;
        case 3: go(bf, std::integral_constant<int, 3>{}); break;
        case 4: go(bf, std::integral_constant<int, 4>{}); break;
        default: go(bf, std::integral_constant<int, 0>{}); break;
      }
    };
    if (x_bf16)
      go_s(std::true_type{});
    else
      go_s(std::false_type{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!budget_in && t <= kSmallT)
    hipLaunchKernelGGL(route_small_kernel, dim3(1), dim3(64), 0, stream, t, s, logits, budget,
                       perm, offsets);
  else
    hipLaunchKernelGGL(route_kernel, dim3(1), dim3(1024), 0, stream, t, s,
                       budget_in ? nullptr : logits, budget_in, budget, perm, offsets);
  return hipGetLastError();
}

}  // namespace mbq
