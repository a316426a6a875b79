// Routed prefill linear (T > 64): per budget group b, Y_b = X_b . W^(b)^T with
// W^(b) = sum_{j <= b} deq(Q_j) dequantized to bfloat16 in LDS and fed to MFMA.
//
// MoBiQuant explainer (gist.science, English), sections 2.A and 4: the summed slices are
// the token's weight, and prefill latency grows linearly with sequence length, i.e. the
// path is a dense contraction.  The pages' own kernel uses 1-bit binary tensor-core MMA on
// another vendor's GPU; CDNA4 has no 1-bit MFMA, so here the slices are summed in float32
// registers, rounded once to bfloat16 and multiplied on bf16 MFMA with float32
// accumulation.  float32 activations are rounded to bfloat16 on the way into LDS.
//
// Tokens arrive sorted by budget (perm, offsets); every M tile holds tokens of a single
// budget, so each group's tiles are padded to the tile height and the grid has at most
// S - 1 more M tiles than ceil(T / BM).  A rows are gathered through perm; the epilogue
// scatters back to the original token order.
#include "mbq_internal.h"

namespace mbq {
namespace {

constexpr int BM = 128, BN = 128, BK = 64, LDS_STRIDE = BK + 8;  // bf16 elements per row

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <bool XBF16>
__global__ __launch_bounds__(256) void prefill_kernel(
    const uint8_t* __restrict__ packed, int N, int K, int G, int KB, int NG, int NB, int S,
    uint64_t slice_stride, uint64_t params_offset, const void* __restrict__ x, int T,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets, void* __restrict__ y,
    int y_bf16) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDS_STRIDE];

  // Which budget group and which tokens this M tile covers.
  int m = blockIdx.y, b = 0, start = 0, rows = 0;
  for (int bb = 1; bb <= S; ++bb) {
    // offsets out of contract are clamped into [0, T] so no tile reaches past perm
    const int lo = min(max(offsets[bb - 1], 0), T), hi = min(max(offsets[bb], lo), T);
    const int nt = (hi - lo + BM - 1) / BM;
    if (m < nt) {
      b = bb;
      start = lo + m * BM;
      rows = min(BM, hi - start);
      break;
    }
    m -= nt;
  }
  if (b == 0) return;  // uniform over the workgroup

  const int n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  // A staging: thread -> (row tid/2, 32 inputs at 32*(tid%2))
  const int arow = tid >> 1, acol = (tid & 1) * 32;
  const int pa = arow < rows ? perm[start + arow] : -1;
  const int src = (pa >= 0 && pa < T) ? pa : -1;
  // B staging: thread -> row block tid/32 of the tile, tile lanes 2*(tid%32) + {0, 1}
  const int brb = tid >> 5;
  const int bnb = n0 / 16 + brb;

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += BK) {
    // ---- A tile: gather token rows, round to bf16
    {
      uint32_t pk[16];
      if (src >= 0 && k0 + acol < K) {   // K is a multiple of 32: the 32 inputs are all in or all past
        if (XBF16) {
          const u32x4_t* p = reinterpret_cast<const u32x4_t*>(
              static_cast<const uint16_t*>(x) + size_t(src) * K + k0 + acol);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4_t v = p[q];
            pk[4 * q] = v[0]; pk[4 * q + 1] = v[1]; pk[4 * q + 2] = v[2]; pk[4 * q + 3] = v[3];
          }
        } else {
          const f32x4_t* p = reinterpret_cast<const f32x4_t*>(
              static_cast<const float*>(x) + size_t(src) * K + k0 + acol);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const f32x4_t v = p[q];
            pk[2 * q] = bf16_bits_rne(v[0]) | (bf16_bits_rne(v[1]) << 16);
            pk[2 * q + 1] = bf16_bits_rne(v[2]) | (bf16_bits_rne(v[3]) << 16);
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) pk[q] = 0u;
      }
      u32x4_t* d = reinterpret_cast<u32x4_t*>(As + arow * LDS_STRIDE + acol);
#pragma unroll
      for (int q = 0; q < 4; ++q) d[q] = u32x4_t{pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]};
    }
    // ---- B tile: W^(b) for 128 rows x 64 inputs, summed in float32, rounded to bf16
    {
      const int kb = k0 >> 8, wi = (k0 & 255) >> 6;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int L = 2 * (tid & 31) + u;
        const int r = L & 15, c = L >> 4;
        const int g = (k0 + 16 * c) / G;   // the lane's 16 inputs lie in one group (G >= 32)
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = 0.f;
        if (bnb < NB) {
          for (int j = 0; j < b; ++j) {
            const uint8_t* sl = packed + uint64_t(j) * slice_stride;
            const uint32_t w = *reinterpret_cast<const uint32_t*>(sl + (size_t(bnb) * KB + kb) * kTileBytes + 16 * L + 4 * wi);
            const uint32_t pv = *reinterpret_cast<const uint32_t*>(sl + params_offset + ((size_t(bnb) * NG + g) * 16 + r) * 4);
            const float s = __half2float(__ushort_as_half(uint16_t(pv & 0xFFFFu)));
            const float z = __half2float(__ushort_as_half(uint16_t(pv >> 16)));
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] += fmaf(s, float((w >> (16 * (e & 1) + 2 * (e >> 1))) & 3u), z);
          }
        }
        uint32_t pk[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pk[e] = bf16_bits_rne(v[2 * e]) | (bf16_bits_rne(v[2 * e + 1]) << 16);
        u32x4_t* d = reinterpret_cast<u32x4_t*>(Bs + (16 * brb + r) * LDS_STRIDE + 16 * c);
        d[0] = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
        d[1] = u32x4_t{pk[4], pk[5], pk[6], pk[7]};
      }
    }
    __syncthreads();
    // ---- MFMA: each wave owns a 64 x 64 quadrant of the 128 x 128 tile
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      u32x4_t a[4], bv[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        a[mi] = *reinterpret_cast<const u32x4_t*>(As + (64 * wm + 16 * mi + (lane & 15)) * LDS_STRIDE + kk + 8 * (lane >> 4));
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        bv[ni] = *reinterpret_cast<const u32x4_t*>(Bs + (64 * wn + 16 * ni + (lane & 15)) * LDS_STRIDE + kk + 8 * (lane >> 4));
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma(a[mi], bv[ni], acc[mi][ni]);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds tokens 4*(lane/16) + v of each 16-row block, row lane%16
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 64 * wm + 16 * mi + 4 * (lane >> 4) + v;
      if (row >= rows) continue;
      const int tok = perm[start + row];
      if (tok < 0 || tok >= T) continue;
      const size_t ybase = size_t(tok) * N;
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int n = n0 + 64 * wn + 16 * ni + (lane & 15);
        if (n < N) {
          if (y_bf16)
            reinterpret_cast<uint16_t*>(y)[ybase + n] = uint16_t(bf16_bits_rne(acc[mi][ni][v]));
          else
            reinterpret_cast<float*>(y)[ybase + n] = acc[mi][ni][v];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(const mbq_desc& d, const void* packed, int32_t t, const void* x,
                          bool x_bf16, const int32_t* perm, const int32_t* offsets, void* y,
                          bool y_bf16, hipStream_t stream) {
  dim3 grid((d.n + BN - 1) / BN, (t + BM - 1) / BM + d.slices - 1), block(256);
  const auto* pk = static_cast<const uint8_t*>(packed);
  if (x_bf16)
    hipLaunchKernelGGL(prefill_kernel<true>, grid, block, 0, stream, pk, d.n, d.k, d.group,
                       d.k_tiles, d.groups_padded, d.row_blocks, d.slices, d.slice_stride,
                       d.params_offset, x, t, perm, offsets, y, int(y_bf16));
  else
    hipLaunchKernelGGL(prefill_kernel<false>, grid, block, 0, stream, pk, d.n, d.k, d.group,
                       d.k_tiles, d.groups_padded, d.row_blocks, d.slices, d.slice_stride,
                       d.params_offset, x, t, perm, offsets, y, int(y_bf16));
  return hipGetLastError();
}

}  // namespace mbq
