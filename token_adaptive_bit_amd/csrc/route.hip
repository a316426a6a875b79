// MoBiRoute, linear-argmax form, and the token regroup.
//
// MoBiQuant explainer (gist.science, English), section 2.B: a lightweight router scores
// each token and the scores decide how many residual slices the token activates.  Here
// the score is logits = x . Wr (float32 accumulate) and b(t) = 1 + the first index of the
// largest logit.  Tokens are then regrouped by a stable ascending sort on b(t) so that
// the linear kernels see runs of tokens with one budget (the pages leave the regroup
// open; the English page, section 5, names irregular access as the cost it avoids).
#include "mbq_internal.h"

namespace mbq {
namespace {

// One wave per token: lanes stride over K, then a butterfly sum.  Deterministic.
template <bool BF16>
__global__ __launch_bounds__(256) void logits_kernel(const void* __restrict__ x, int T, int K,
                                                     int S, const float* __restrict__ wr,
                                                     float* __restrict__ logits) {
  const int t = blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x & 63;
  if (t >= T) return;  // whole waves exit together
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k = lane; k < K; k += 64) {
    const float xv = load_x(x, size_t(t) * K + k, BF16);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if (s < S) acc[s] = fmaf(xv, wr[size_t(k) * S + s], acc[s]);
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    float v = acc[s];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    if (s < S && lane == 0) logits[size_t(t) * S + s] = v;
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
    const float* l = logits + size_t(t) * S;
    float best = l[0];
    int arg = 0;
    for (int j = 1; j < S; ++j)
      if (l[j] > best) { best = l[j]; arg = j; }
    return arg + 1;
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
    dim3 grid((t + 3) / 4), block(256);
    if (x_bf16)
      hipLaunchKernelGGL(logits_kernel<true>, grid, block, 0, stream, x, t, k, s, wr, logits);
    else
      hipLaunchKernelGGL(logits_kernel<false>, grid, block, 0, stream, x, t, k, s, wr, logits);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(1024), 0, stream, t, s,
                     budget_in ? nullptr : logits, budget_in, budget, perm, offsets);
  return hipGetLastError();
}

}  // namespace mbq
