// MoBiSlice pack: recursive 2-bit residual quantization into the slice-major blob.
//
// MoBiQuant explainer (gist.science, English), section 2.A: the first slice quantizes W,
// each later slice quantizes the residual left by the previous ones, and a precision of
// b slices is the sum of the first b.  The quantizer is the 2-bit asymmetric min/max
// round-to-nearest reading documented in mbq.h.
//
// One wave per packed tile (16 rows x 256 inputs).  Lane l = 16c + r owns row r of the
// tile and inputs 64i + 16c + e (i = 0..3, e = 0..15): exactly the 64 codes it stores as
// one 16-byte vector, so the codes of every slice leave the kernel as one coalesced
// 1 KiB store per wave.  A group of G >= 64 inputs of one row is spread over the 4 lanes
// r, r+16, r+32, r+48 (G/64 words each), so its min and max need two cross-lane steps; a
// group of 32 is word i of the lane pair c = 2h, 2h+1 (group 2i + h of the tile) and
// needs one.
// The residual of all 64 inputs stays in registers across the slices.
//
// Bit-exactness: every float32 operation is rounded on its own (this file is built with
// -ffp-contract=off and uses the _rn intrinsics), division is IEEE, rint rounds half to
// even and float->half rounds to nearest even with subnormals.
#include "mbq_internal.h"

namespace mbq {
namespace {

// w holds the N rows being packed; they land in row blocks nb0 .. of a blob of NBT row
// blocks (a part of a larger weight when nb0 > 0 or N < 16 NBT: groups are per row, so
// packing rows on their own gives the same codes as packing them with their neighbours).
template <int G, bool BF16>
__global__ __launch_bounds__(64) void pack_kernel(const void* __restrict__ w, int N, int K,
                                                  int S, int KB, int NG, uint64_t slice_stride,
                                                  uint64_t params_offset, int nb0, int NBT,
                                                  uint8_t* __restrict__ packed,
                                                  int32_t* __restrict__ status) {
  // G = 32: one pass per word, each lane pair holding a group of its own
  constexpr bool kPair = G == 32;
  constexpr int kWordsPerGroup = kPair ? 1 : G / 64;
  constexpr int kGroupsPerTile = 256 / G;
  constexpr int kPasses = kPair ? 4 : kGroupsPerTile;
  const int kb = blockIdx.x, nb = nb0 + blockIdx.y;
  const int lane = threadIdx.x, r = lane & 15, c = lane >> 4;
  const int n = blockIdx.y * 16 + r;  // row of w

  float R[4][16];
  int bad = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int k = kb * 256 + 64 * i + 16 * c + e;
      float v = 0.f;
      if (n < N && k < K) v = load_x(w, size_t(n) * K + k, BF16);
      if (!__builtin_isfinite(v)) bad |= 1;
      R[i][e] = v;
    }
  }

  for (int j = 0; j < S; ++j) {
    uint8_t* slice = packed + uint64_t(j) * slice_stride;
    uint32_t word[4];
#pragma unroll
    for (int gi = 0; gi < kPasses; ++gi) {
      float lo = R[gi * kWordsPerGroup][0], hi = lo;
#pragma unroll
      for (int ii = 0; ii < kWordsPerGroup; ++ii) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          lo = fminf(lo, R[gi * kWordsPerGroup + ii][e]);
          hi = fmaxf(hi, R[gi * kWordsPerGroup + ii][e]);
        }
      }
      lo = fminf(lo, __shfl_xor(lo, 16));
      hi = fmaxf(hi, __shfl_xor(hi, 16));
      if (!kPair) {
        lo = fminf(lo, __shfl_xor(lo, 32));
        hi = fmaxf(hi, __shfl_xor(hi, 32));
      }
      lo = __fadd_rn(lo, 0.0f);  // a signed-zero minimum is stored as +0
      const float span = __fsub_rn(hi, lo);
      const float step = __fdiv_rn(span, 3.0f);
      // float -> half rounds to infinity from 65520 on (round to nearest even)
      if (!(fabsf(step) < 65520.f) || !(fabsf(lo) < 65520.f)) bad |= 2;
      const __half hs = __float2half_rn(step);
      const __half hz = __float2half_rn(lo);
      const float sf = __half2float(hs);
      const float zf = __half2float(hz);
#pragma unroll
      for (int ii = 0; ii < kWordsPerGroup; ++ii) {
        const int i = gi * kWordsPerGroup + ii;
        uint32_t wd = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float rv = R[i][e];
          float q = 0.f;
          if (sf != 0.f) {
            const float u = __fdiv_rn(__fsub_rn(rv, zf), sf);
            q = fminf(fmaxf(rintf(u), 0.f), 3.f);
          }
          wd |= uint32_t(q) << (16 * (e & 1) + 2 * (e >> 1));  // even e: low half, odd e: high half
          const float dq = __fadd_rn(zf, __fmul_rn(q, sf));
          R[i][e] = __fsub_rn(rv, dq);
        }
        word[i] = wd;
      }
      if (kPair ? (c & 1) == 0 : c == 0) {
        const uint32_t pv = uint32_t(__half_as_ushort(hs)) | (uint32_t(__half_as_ushort(hz)) << 16);
        const size_t g = size_t(kb) * kGroupsPerTile + (kPair ? 2 * gi + (c >> 1) : gi);
        *reinterpret_cast<uint32_t*>(slice + params_offset + ((size_t(nb) * NG + g) * 16 + r) * 4) = pv;
      }
    }
    u32x4_t v = {word[0], word[1], word[2], word[3]};
    *reinterpret_cast<u32x4_t*>(slice + (size_t(nb) * KB + kb) * kTileBytes + 16 * lane) = v;
  }
  // The wave of the blob's last row block and first k tile also clears each slice's
  // alignment gap after its params, so that the whole blob is defined.
  if (kb == 0 && nb == NBT - 1) {
    const uint64_t used = params_offset + uint64_t(NBT) * NG * 64;
    for (int j = 0; j < S; ++j)
      for (uint64_t off = used + 4 * lane; off < slice_stride; off += 256)
        *reinterpret_cast<uint32_t*>(packed + uint64_t(j) * slice_stride + off) = 0u;
  }
  if (bad && status) atomicOr(status, bad);
}

// Bit-plane slices (the other reading of "an MSB slice plus residual slices"): one
// uniform 2S-bit min/max code per weight, 4^S levels with step = half(span / (4^S - 1))
// and zero = half(min); slice j stores the code's j-th 2-bit plane from the top with
// scale step * 4^(S-j) and a zero that centres every b-plane prefix sum over the planes
// it drops: zero_1 = half(min + c_1), zero_j = half(c_j - c_(j-1)), c_b = step (4^(S-b) - 1) / 2.
// Same tile and lane layout as pack_kernel; every float32 operation rounded on its own.
template <int G, bool BF16>
__global__ __launch_bounds__(64) void pack_bitplane_kernel(const void* __restrict__ w, int N, int K,
                                                           int S, int KB, int NG, uint64_t slice_stride,
                                                           uint64_t params_offset, int NBT,
                                                           uint8_t* __restrict__ packed,
                                                           int32_t* __restrict__ status) {
  constexpr bool kPair = G == 32;
  constexpr int kWordsPerGroup = kPair ? 1 : G / 64;
  constexpr int kGroupsPerTile = 256 / G;
  constexpr int kPasses = kPair ? 4 : kGroupsPerTile;
  const int kb = blockIdx.x, nb = blockIdx.y;
  const int lane = threadIdx.x, r = lane & 15, c = lane >> 4;
  const int n = nb * 16 + r;
  const float levels = float((1 << (2 * S)) - 1);

  // W of this lane's 64 inputs; replaced in place by the full codes q (small integers)
  float V[4][16];
  int bad = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int k = kb * 256 + 64 * i + 16 * c + e;
      float v = 0.f;
      if (n < N && k < K) v = load_x(w, size_t(n) * K + k, BF16);
      if (!__builtin_isfinite(v)) bad |= 1;
      V[i][e] = v;
    }
  float sfv[kPasses], zfv[kPasses];
#pragma unroll
  for (int gi = 0; gi < kPasses; ++gi) {
    float lo = V[gi * kWordsPerGroup][0], hi = lo;
#pragma unroll
    for (int ii = 0; ii < kWordsPerGroup; ++ii)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        lo = fminf(lo, V[gi * kWordsPerGroup + ii][e]);
        hi = fmaxf(hi, V[gi * kWordsPerGroup + ii][e]);
      }
    lo = fminf(lo, __shfl_xor(lo, 16));
    hi = fmaxf(hi, __shfl_xor(hi, 16));
    if (!kPair) {
      lo = fminf(lo, __shfl_xor(lo, 32));
      hi = fmaxf(hi, __shfl_xor(hi, 32));
    }
    lo = __fadd_rn(lo, 0.0f);  // a signed-zero minimum is stored as +0
    const float step = __fdiv_rn(__fsub_rn(hi, lo), levels);
    const float sf = __half2float(__float2half_rn(step));
    const float zf = __half2float(__float2half_rn(lo));
    sfv[gi] = sf;
    zfv[gi] = zf;
#pragma unroll
    for (int ii = 0; ii < kWordsPerGroup; ++ii)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int i = gi * kWordsPerGroup + ii;
        float q = 0.f;
        if (sf != 0.f) q = fminf(fmaxf(rintf(__fdiv_rn(__fsub_rn(V[i][e], zf), sf)), 0.f), levels);
        V[i][e] = q;
      }
  }
  for (int j = 0; j < S; ++j) {
    uint8_t* slice = packed + uint64_t(j) * slice_stride;
    const int shift = 2 * (S - 1 - j);
    uint32_t word[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t wd = 0;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t p = (uint32_t(V[i][e]) >> shift) & 3u;
        wd |= p << (16 * (e & 1) + 2 * (e >> 1));
      }
      word[i] = wd;
    }
#pragma unroll
    for (int gi = 0; gi < kPasses; ++gi) {
      const float sf = sfv[gi];
      // slice b = j + 1: 4^(S-b) = 2^shift; c_b and c_(b-1) (the latter used for b > 1)
      const float cj = __fmul_rn(sf, float((1 << shift) - 1) * 0.5f);
      const float cp = __fmul_rn(sf, float((1 << (shift + 2)) - 1) * 0.5f);
      const __half hs = __float2half_rn(__fmul_rn(sf, float(1 << shift)));
      const __half hz = __float2half_rn(j == 0 ? __fadd_rn(zfv[gi], cj) : __fsub_rn(cj, cp));
      if (__hisinf(hs) || __hisinf(hz) || __hisnan(hs) || __hisnan(hz)) bad |= 2;
      if (kPair ? (c & 1) == 0 : c == 0) {
        const uint32_t pv = uint32_t(__half_as_ushort(hs)) | (uint32_t(__half_as_ushort(hz)) << 16);
        const size_t g = size_t(kb) * kGroupsPerTile + (kPair ? 2 * gi + (c >> 1) : gi);
        *reinterpret_cast<uint32_t*>(slice + params_offset + ((size_t(nb) * NG + g) * 16 + r) * 4) = pv;
      }
    }
    u32x4_t v = {word[0], word[1], word[2], word[3]};
    *reinterpret_cast<u32x4_t*>(slice + (size_t(nb) * KB + kb) * kTileBytes + 16 * lane) = v;
  }
  if (kb == 0 && nb == NBT - 1) {
    const uint64_t used = params_offset + uint64_t(NBT) * NG * 64;
    for (int j = 0; j < S; ++j)
      for (uint64_t off = used + 4 * lane; off < slice_stride; off += 256)
        *reinterpret_cast<uint32_t*>(packed + uint64_t(j) * slice_stride + off) = 0u;
  }
  if (bad && status) atomicOr(status, bad);
}

template <int G>
hipError_t launch_bp(const mbq_desc& d, const void* w, bool w_bf16, void* packed, int32_t* st,
                     hipStream_t stream) {
  dim3 grid(d.k_tiles, d.row_blocks), block(64);
  auto* out = static_cast<uint8_t*>(packed);
  if (w_bf16)
    hipLaunchKernelGGL((pack_bitplane_kernel<G, true>), grid, block, 0, stream, w, d.n, d.k, d.slices,
                       d.k_tiles, d.groups_padded, d.slice_stride, d.params_offset, d.row_blocks, out, st);
  else
    hipLaunchKernelGGL((pack_bitplane_kernel<G, false>), grid, block, 0, stream, w, d.n, d.k, d.slices,
                       d.k_tiles, d.groups_padded, d.slice_stride, d.params_offset, d.row_blocks, out, st);
  return hipGetLastError();
}

template <int G>
hipError_t launch_g(const mbq_desc& d, int32_t row0, int32_t rows, const void* w, bool w_bf16,
                    void* packed, int32_t* st, hipStream_t stream) {
  dim3 grid(d.k_tiles, (rows + 15) / 16), block(64);
  auto* out = static_cast<uint8_t*>(packed);
  const int nb0 = row0 / 16;
  if (w_bf16)
    hipLaunchKernelGGL((pack_kernel<G, true>), grid, block, 0, stream, w, rows, d.k, d.slices,
                       d.k_tiles, d.groups_padded, d.slice_stride, d.params_offset, nb0,
                       d.row_blocks, out, st);
  else
    hipLaunchKernelGGL((pack_kernel<G, false>), grid, block, 0, stream, w, rows, d.k, d.slices,
                       d.k_tiles, d.groups_padded, d.slice_stride, d.params_offset, nb0,
                       d.row_blocks, out, st);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_bitplane(const mbq_desc& d, const void* w, bool w_bf16, void* packed,
                                int32_t* st, hipStream_t stream) {
  switch (d.group) {
    case 32: return launch_bp<32>(d, w, w_bf16, packed, st, stream);
    case 64: return launch_bp<64>(d, w, w_bf16, packed, st, stream);
    case 128: return launch_bp<128>(d, w, w_bf16, packed, st, stream);
    default: return launch_bp<256>(d, w, w_bf16, packed, st, stream);
  }
}

hipError_t launch_pack(const mbq_desc& d, int32_t row0, int32_t rows, const void* w, bool w_bf16,
                       void* packed, int32_t* st, hipStream_t stream) {
  switch (d.group) {
    case 32: return launch_g<32>(d, row0, rows, w, w_bf16, packed, st, stream);
    case 64: return launch_g<64>(d, row0, rows, w, w_bf16, packed, st, stream);
    case 128: return launch_g<128>(d, row0, rows, w, w_bf16, packed, st, stream);
    default: return launch_g<256>(d, row0, rows, w, w_bf16, packed, st, stream);
  }
}

}  // namespace mbq
