// Internal declarations of libmbq: kernel launchers and small device helpers.
// Everything here is gfx950 (CDNA4, wave64) code; nothing is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/mbq.h"

namespace mbq {

constexpr int kWave = 64;
constexpr int kRowBlock = 16;    // rows per packed tile
constexpr int kKTile = 256;      // inputs per packed tile
constexpr int kTileBytes = 1024; // 16 rows x 256 inputs x 2 bits
constexpr int kMaxLrChunks = 8;  // K chunks of the low-rank side path's u = x A^T

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

// bfloat16 bits of a float, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float load_x(const void* p, size_t idx, bool is_bf16) {
  if (is_bf16) return bf16_bits_to_float(reinterpret_cast<const uint16_t*>(p)[idx]);
  return reinterpret_cast<const float*>(p)[idx];
}

// Host-side launchers (one per translation unit).
hipError_t launch_pack(const mbq_desc& d, int32_t row0, int32_t rows, const void* w, bool w_bf16,
                       void* packed, int32_t* dev_status, hipStream_t stream);
hipError_t launch_pack_bitplane(const mbq_desc& d, const void* w, bool w_bf16, void* packed,
                                int32_t* dev_status, hipStream_t stream);
hipError_t launch_route(int32_t t, int32_t k, int32_t s, const void* x, bool x_bf16,
                        const float* wr, float* logits, const int32_t* budget_in,
                        int32_t* budget, int32_t* perm, int32_t* offsets, hipStream_t stream);
size_t route_mlp_workspace(int32_t t, int32_t k, int32_t h);
hipError_t launch_route_mlp(int32_t t, int32_t k, int32_t s, int32_t h, const void* x, bool x_bf16,
                            const uint16_t* w1, const float* b1, const float* w2, const float* b2,
                            float theta, float* scores, int32_t* budget, int32_t* perm,
                            int32_t* offsets, void* ws, hipStream_t stream);
size_t decode_workspace(const mbq_desc& d, int32_t t, bool x_bf16);
hipError_t launch_decode(const mbq_desc& d, const void* packed, int32_t t, const void* x,
                         bool x_bf16, const int32_t* perm, const int32_t* offsets, void* y,
                         bool y_bf16, void* ws, hipStream_t stream);
bool decode_stream_supported(const mbq_desc& d, int32_t t, bool x_bf16, bool lr = false);
size_t decode_stream_workspace(const mbq_desc& d, int32_t t, bool x_bf16, bool lr);
bool decode_stream_lr_inline(const mbq_desc& d, int32_t t, bool x_bf16);
// The low-rank side path's call state at the front of its workspace, where the streaming
// decode computes u inside its launch: 256 bytes of words (launch count, error flags),
// one 128-byte check-in line for each of at most kLrMaxWg workgroups (from byte 256),
// then u of every 16-token block as 8-byte pairs (from byte kLrPairs, rounded up to 256
// bytes).  The offsets do not depend on t, so calls of any size can share a workspace.
constexpr int kLrMaxWg = 512;
constexpr size_t kLrSlots = 256, kLrPairs = kLrSlots + size_t(kLrMaxWg) * 128;
inline size_t lr_state_bytes(int32_t t, int32_t rank) {
  return kLrPairs + (size_t((t + 15) / 16) * 16 * size_t(rank) * 8 + 255) / 256 * 256;
}
// Decode with the routing in the kernel (bfloat16 x, 1 <= t <= 16, K within one
// workgroup): writes logits, budget, perm and offsets as launch_route does, and y.
bool decode_route_supported(const mbq_desc& d, int32_t t);
// mul: an mbq_mul (MBQ_MUL_AUTO lets the plan choose); launches: 0 (the plan's choice), 1
// or 2.  The fp8 x fp4 step runs as two launches (the prepared operands in ws, which must
// then hold decode_route_workspace() bytes) when asked to or, by default, above 8 tokens
// with that much workspace; otherwise as one.
size_t decode_route_workspace(const mbq_desc& d, int32_t t);
// The two launches apart: the prepared operands (decode_prep_kernel), and the streaming
// kernel that routes from their partial logits.  Blobs of 2 or more slices.
bool decode_prepared_supported(const mbq_desc& d, int32_t t);
hipError_t launch_decode_prepare(const mbq_desc& d, int32_t t, const void* x, const float* wr, void* prep,
                                 hipStream_t stream);
hipError_t launch_decode_prepared(const mbq_desc& d, const void* packed, int32_t t, const void* prep,
                                  float* logits, int32_t* budget, int32_t* perm, int32_t* offsets, void* y,
                                  bool y_bf16, hipStream_t stream);
hipError_t launch_decode_route(const mbq_desc& d, const void* packed, int32_t t, const void* x,
                               const float* wr, float* logits, int32_t* budget, int32_t* perm,
                               int32_t* offsets, void* y, bool y_bf16, int mul, int launches, void* ws,
                               size_t ws_bytes, hipStream_t stream);
hipError_t launch_decode_stream(const mbq_desc& d, const void* packed, int32_t t, const void* x,
                                bool x_bf16, const int32_t* perm, const int32_t* offsets,
                                void* y, bool y_bf16, void* ws, const float* lr_u, int32_t lr_ks,
                                const uint16_t* lr_b, int32_t lr_r, uint8_t* lr_fz,
                                const uint16_t* lr_a, hipStream_t stream);
hipError_t launch_prefill(const mbq_desc& d, const void* packed, int32_t t, const void* x,
                          bool x_bf16, const int32_t* perm, const int32_t* offsets, void* y,
                          bool y_bf16, hipStream_t stream);
bool prefill_mfma_supported(const mbq_desc& d, int32_t t, const void* x, bool x_bf16);
// slots: workgroups the tile plan assumes run at once (0: the device's compute units).
hipError_t launch_prefill_mfma(const mbq_desc& d, const void* packed, int32_t t, const void* x,
                               bool x_bf16, const int32_t* perm, const int32_t* offsets, void* y,
                               bool y_bf16, const float* lr_u, int32_t lr_ks, const uint16_t* lr_b,
                               int32_t lr_r, int32_t slots, hipStream_t stream);
hipError_t launch_lowrank_u(int32_t t, int32_t k, const void* x, bool x_bf16, const uint16_t* a,
                            int32_t rank, float* u, hipStream_t stream);
int lowrank_u_chunks(int32_t t, int32_t k);
hipError_t launch_lowrank_update(int32_t t, int32_t n, const float* u, int32_t ksu, const uint16_t* b,
                                 int32_t rank, void* y, bool y_bf16, hipStream_t stream);

}  // namespace mbq
