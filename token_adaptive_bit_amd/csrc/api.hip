// Host side of the C ABI: validation, geometry, dispatch.  No device work happens here
// until every argument has been checked, so all error paths run without a GPU.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "mbq_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

bool valid_dtype(mbq_dtype t) { return t == MBQ_F32 || t == MBQ_BF16; }

mbq_status check_desc(const mbq_desc* d) {
  if (!d) return MBQ_ERR_ARG;
  if (d->abi != MBQ_ABI_VERSION || d->bits != 2) return MBQ_ERR_UNSUPPORTED;
  mbq_desc ref;
  mbq_status st = mbq_describe(d->n, d->k, d->group, d->slices, &ref);
  if (st != MBQ_OK) return st;
  if (ref.total_bytes != d->total_bytes || ref.slice_stride != d->slice_stride ||
      ref.params_offset != d->params_offset || ref.row_blocks != d->row_blocks ||
      ref.k_tiles != d->k_tiles || ref.groups_padded != d->groups_padded)
    return MBQ_ERR_SHAPE;
  return MBQ_OK;
}

// With MBQ_DEBUG set in the environment, a failed launch also prints the HIP error.
mbq_status launched(hipError_t e) {
  if (e == hipSuccess) e = hipGetLastError();
  if (e == hipSuccess) return MBQ_OK;
  if (std::getenv("MBQ_DEBUG")) std::fprintf(stderr, "libmbq: launch failed: %s (%d)\n", hipGetErrorString(e), int(e));
  return MBQ_ERR_DEVICE;
}

}  // namespace

extern "C" {

int32_t mbq_abi_version(void) { return MBQ_ABI_VERSION; }

const char* mbq_status_str(mbq_status s) {
  switch (s) {
    case MBQ_OK: return "ok";
    case MBQ_ERR_ARG: return "invalid argument (NULL or misaligned pointer, unknown dtype)";
    case MBQ_ERR_SHAPE: return "invalid shape";
    case MBQ_ERR_RANGE: return "value out of range";
    case MBQ_ERR_WORKSPACE: return "workspace missing or too small";
    case MBQ_ERR_DEVICE: return "HIP launch failed";
    case MBQ_ERR_UNSUPPORTED: return "unsupported group, slice count, bit width or ABI version";
  }
  return "unknown status";
}

mbq_status mbq_describe(int32_t n, int32_t k, int32_t group, int32_t slices, mbq_desc* out) {
  if (!out) return MBQ_ERR_ARG;
  if (group != 32 && group != 64 && group != 128 && group != 256) return MBQ_ERR_UNSUPPORTED;
  if (slices < 1 || slices > 4) return MBQ_ERR_UNSUPPORTED;
  if (n < 1 || k < group || (k % group) != 0) return MBQ_ERR_SHAPE;
  if (n > (1 << 28) || k > (1 << 28)) return MBQ_ERR_SHAPE;
  mbq_desc d{};
  d.abi = MBQ_ABI_VERSION;
  d.n = n;
  d.k = k;
  d.group = group;
  d.slices = slices;
  d.bits = 2;
  d.row_blocks = (n + mbq::kRowBlock - 1) / mbq::kRowBlock;
  d.k_tiles = (k + mbq::kKTile - 1) / mbq::kKTile;
  d.groups_padded = d.k_tiles * mbq::kKTile / group;
  d.codes_bytes = uint64_t(d.row_blocks) * d.k_tiles * mbq::kTileBytes;
  d.params_bytes = uint64_t(d.row_blocks) * d.groups_padded * 64;
  d.params_offset = align256(d.codes_bytes);
  d.slice_stride = d.params_offset + align256(d.params_bytes);
  d.total_bytes = d.slice_stride * uint64_t(slices);
  *out = d;
  return MBQ_OK;
}

mbq_status mbq_pack(const mbq_desc* desc, const void* w, mbq_dtype w_dtype, void* packed,
                    int32_t* dev_status, hipStream_t stream) {
  mbq_status st = check_desc(desc);
  if (st != MBQ_OK) return st;
  if (!valid_dtype(w_dtype) || !w || !packed) return MBQ_ERR_ARG;
  if (!aligned(packed, 256) || !aligned(w, w_dtype == MBQ_F32 ? 4 : 2)) return MBQ_ERR_ARG;
  if (dev_status && !aligned(dev_status, 4)) return MBQ_ERR_ARG;
  return launched(mbq::launch_pack(*desc, 0, desc->n, w, w_dtype == MBQ_BF16, packed, dev_status,
                                   stream));
}

mbq_status mbq_pack_bitplane(const mbq_desc* desc, const void* w, mbq_dtype w_dtype, void* packed,
                             int32_t* dev_status, hipStream_t stream) {
  mbq_status st = check_desc(desc);
  if (st != MBQ_OK) return st;
  if (!valid_dtype(w_dtype) || !w || !packed) return MBQ_ERR_ARG;
  if (!aligned(packed, 256) || !aligned(w, w_dtype == MBQ_F32 ? 4 : 2)) return MBQ_ERR_ARG;
  if (dev_status && !aligned(dev_status, 4)) return MBQ_ERR_ARG;
  return launched(mbq::launch_pack_bitplane(*desc, w, w_dtype == MBQ_BF16, packed, dev_status, stream));
}

mbq_status mbq_pack_rows(const mbq_desc* desc, int32_t row0, int32_t rows, const void* w,
                         mbq_dtype w_dtype, void* packed, int32_t* dev_status, hipStream_t stream) {
  mbq_status st = check_desc(desc);
  if (st != MBQ_OK) return st;
  if (!valid_dtype(w_dtype) || !w || !packed) return MBQ_ERR_ARG;
  if (!aligned(packed, 256) || !aligned(w, w_dtype == MBQ_F32 ? 4 : 2)) return MBQ_ERR_ARG;
  if (dev_status && !aligned(dev_status, 4)) return MBQ_ERR_ARG;
  // whole row blocks only: a part starts on a block and fills its blocks unless it ends the blob
  if (row0 < 0 || rows < 1 || row0 % 16 != 0 || int64_t(row0) + rows > desc->n) return MBQ_ERR_SHAPE;
  if (rows % 16 != 0 && row0 + rows != desc->n) return MBQ_ERR_SHAPE;
  return launched(mbq::launch_pack(*desc, row0, rows, w, w_dtype == MBQ_BF16, packed, dev_status,
                                   stream));
}

mbq_status mbq_route(int32_t t, int32_t k, int32_t s, const void* x, mbq_dtype x_dtype,
                     const float* wr, float* logits, int32_t* budget, int32_t* perm,
                     int32_t* offsets, hipStream_t stream) {
  if (s < 1 || s > 4) return MBQ_ERR_UNSUPPORTED;
  if (t < 0 || t > (1 << 24)) return MBQ_ERR_SHAPE;
  if (!offsets) return MBQ_ERR_ARG;
  if (t > 0 && (!logits || !budget || !perm)) return MBQ_ERR_ARG;  // may be NULL when t == 0
  if (x && t > 0) {
    if (k < 1) return MBQ_ERR_SHAPE;
    if (!valid_dtype(x_dtype) || !wr) return MBQ_ERR_ARG;
    if (!aligned(x, x_dtype == MBQ_F32 ? 4 : 2) || !aligned(wr, 4)) return MBQ_ERR_ARG;
  }
  if (!aligned(logits, 4) || !aligned(budget, 4) || !aligned(perm, 4) || !aligned(offsets, 4))
    return MBQ_ERR_ARG;
  return launched(mbq::launch_route(t, k, s, x, x_dtype == MBQ_BF16, wr, logits, nullptr,
                                    budget, perm, offsets, stream));
}

mbq_status mbq_regroup(int32_t t, int32_t s, const int32_t* budget, int32_t* perm,
                       int32_t* offsets, hipStream_t stream) {
  if (s < 1 || s > 4) return MBQ_ERR_UNSUPPORTED;
  if (t < 0 || t > (1 << 24)) return MBQ_ERR_SHAPE;
  if (!offsets || (t > 0 && (!budget || !perm))) return MBQ_ERR_ARG;
  if (!aligned(budget, 4) || !aligned(perm, 4) || !aligned(offsets, 4)) return MBQ_ERR_ARG;
  return launched(mbq::launch_route(t, 0, s, nullptr, false, nullptr, nullptr, budget,
                                    nullptr, perm, offsets, stream));
}

namespace {
bool mlp_shape_ok(int32_t t, int32_t k, int32_t hidden) {
  return t >= 0 && t <= (1 << 24) && k >= 1 && hidden >= 64 && hidden <= 4096 && hidden % 64 == 0;
}
}  // namespace

mbq_status mbq_route_mlp_workspace(int32_t t, int32_t k, int32_t hidden, size_t* bytes) {
  if (!bytes) return MBQ_ERR_ARG;
  if (!mlp_shape_ok(t, k, hidden)) return MBQ_ERR_SHAPE;
  *bytes = mbq::route_mlp_workspace(t, k, hidden);
  return MBQ_OK;
}

mbq_status mbq_route_mlp(int32_t t, int32_t k, int32_t s, int32_t hidden, const void* x,
                         mbq_dtype x_dtype, const uint16_t* w1, const float* b1,
                         const float* w2, const float* b2, double delta, float* scores,
                         int32_t* budget, int32_t* perm, int32_t* offsets, void* workspace,
                         size_t ws_bytes, hipStream_t stream) {
  if (s < 1 || s > 4) return MBQ_ERR_UNSUPPORTED;
  if (t < 0 || t > (1 << 24)) return MBQ_ERR_SHAPE;
  if (std::isnan(delta)) return MBQ_ERR_RANGE;
  if (!offsets) return MBQ_ERR_ARG;
  if (t > 0 && (!budget || !perm || (s > 1 && !scores))) return MBQ_ERR_ARG;
  if (!aligned(scores, 4) || !aligned(budget, 4) || !aligned(perm, 4) || !aligned(offsets, 4))
    return MBQ_ERR_ARG;
  const bool compute = x && t > 0 && s > 1;
  if (compute) {
    if (!mlp_shape_ok(t, k, hidden)) return MBQ_ERR_SHAPE;
    if (!valid_dtype(x_dtype) || !w1 || !b1 || !w2 || !b2) return MBQ_ERR_ARG;
    const size_t esz = x_dtype == MBQ_F32 ? 4 : 2;
    if (!aligned(x, esz) || !aligned(w1, 2) || !aligned(b1, 16) || !aligned(w2, 4) ||
        !aligned(b2, 4))
      return MBQ_ERR_ARG;
    if (size_t(t) * size_t(k) * esz >= (size_t(1) << 31) ||
        size_t(hidden) * size_t(k) * 2 >= (size_t(1) << 31))
      return MBQ_ERR_SHAPE;
    const size_t need = mbq::route_mlp_workspace(t, k, hidden);
    if (need && (!workspace || ws_bytes < need || !aligned(workspace, 16))) return MBQ_ERR_WORKSPACE;
  }
  // theta = logit(delta): sigmoid(score) > delta exactly when score > theta
  double th;
  if (delta <= 0.0)
    th = -HUGE_VAL;
  else if (delta >= 1.0)
    th = HUGE_VAL;
  else
    th = std::log(delta) - std::log1p(-delta);
  return launched(mbq::launch_route_mlp(t, k, s, hidden, compute ? x : nullptr,
                                        x_dtype == MBQ_BF16, w1, b1, w2, b2, float(th), scores,
                                        budget, perm, offsets, workspace, stream));
}

namespace {

// Workspace of the routed linear alone (split-K partials); lr: the side-path plan.
size_t linear_ws(const mbq_desc& d, int32_t t, bool xb, bool lr) {
  size_t n = 0;
  if (t >= 1 && t <= 64) {  // enough for either decode kernel
    n = mbq::decode_workspace(d, t, xb);
    if (mbq::decode_stream_supported(d, t, xb, lr)) n = std::max(n, mbq::decode_stream_workspace(d, t, xb, lr));
  }
  return n;
}

size_t u_bytes(int32_t t, int32_t k, int32_t rank) {
  return align256(uint64_t(mbq::lowrank_u_chunks(t, k)) * uint64_t(t) * uint64_t(rank) * 4);
}

// The side path's call state at the front of its workspace (mbq::lr_state_bytes), used
// where the streaming decode computes u inside its own launch.
size_t lr_state_bytes(int32_t t, int32_t rank) { return mbq::lr_state_bytes(t, rank); }

bool rank_ok(int32_t rank) { return rank >= 8 && rank <= 32 && rank % 8 == 0; }

const mbq_opts kDefaultOpts{};

// NULL means every field 0; a field out of range is an argument error.
const mbq_opts* checked_opts(const mbq_opts* o) {
  if (!o) return &kDefaultOpts;
  if (o->path < MBQ_PATH_AUTO || o->path > MBQ_PATH_GENERIC) return nullptr;
  if (o->decode_mul < MBQ_MUL_AUTO || o->decode_mul > MBQ_MUL_FP8_FP4) return nullptr;
  if (o->prefill_slots < 0 || o->decode_launches < 0 || o->decode_launches > 2) return nullptr;
  return o;
}

bool linear_ptrs_ok(const void* packed, const void* x, const int32_t* perm, const int32_t* offsets,
                    const void* y) {
  return packed && x && perm && offsets && y && aligned(packed, 256) && aligned(x, 16) && aligned(y, 16) &&
         aligned(perm, 4) && aligned(offsets, 4);
}

mbq_status linear_impl(const mbq_desc* desc, const void* packed, int32_t t, const void* x,
                       mbq_dtype x_dtype, const int32_t* perm, const int32_t* offsets,
                       const uint16_t* a, const uint16_t* b, int32_t rank, void* y,
                       mbq_dtype y_dtype, void* workspace, size_t ws_bytes,
                       const mbq_opts* opts_in, hipStream_t stream) {
  mbq_status st = check_desc(desc);
  if (st != MBQ_OK) return st;
  const mbq_opts* opts = checked_opts(opts_in);
  if (!opts) return MBQ_ERR_ARG;
  const bool generic = opts->path == MBQ_PATH_GENERIC;
  if (t < 0 || t > (1 << 24)) return MBQ_ERR_SHAPE;
  if (!valid_dtype(x_dtype) || !valid_dtype(y_dtype)) return MBQ_ERR_ARG;
  if (rank && !rank_ok(rank)) return MBQ_ERR_UNSUPPORTED;
  if (t == 0) return MBQ_OK;  // nothing to compute; t-sized pointers may be NULL
  if (!linear_ptrs_ok(packed, x, perm, offsets, y)) return MBQ_ERR_ARG;
  if (rank && (!a || !b || !aligned(a, 16) || !aligned(b, 16))) return MBQ_ERR_ARG;
  const bool xb = x_dtype == MBQ_BF16, yb = y_dtype == MBQ_BF16, lr = rank > 0;
  // workspace: [side-path state][u partials][the linear's split-K partials]
  const size_t fb = lr ? lr_state_bytes(t, rank) : 0, ub = lr ? u_bytes(t, desc->k, rank) : 0;
  const size_t need = fb + ub + linear_ws(*desc, t, xb, lr);
  const int ksu = lr ? mbq::lowrank_u_chunks(t, desc->k) : 0;
  if (need > 0 && (!workspace || ws_bytes < need || !aligned(workspace, 16)))
    return MBQ_ERR_WORKSPACE;
  uint8_t* fz = lr ? static_cast<uint8_t*>(workspace) : nullptr;
  float* u = lr ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + fb) : nullptr;
  void* lws = need > fb + ub ? static_cast<uint8_t*>(workspace) + fb + ub : nullptr;
  // the generic kernels serve slices of 4 GiB and more (and activations of 4 GiB and more
  // in prefill), which the streaming decode's and the MFMA prefill's 32-bit buffer offsets
  // cannot reach; MBQ_PATH_GENERIC selects them for any size
  const bool streaming = !generic && mbq::decode_stream_supported(*desc, t, xb, lr);
  // the streaming decode computes u inside its own launch where K fits one workgroup
  const bool inline_u = lr && streaming && mbq::decode_stream_lr_inline(*desc, t, xb);
  if (lr && !inline_u) {
    st = launched(mbq::launch_lowrank_u(t, desc->k, x, xb, a, rank, u, stream));
    if (st != MBQ_OK) return st;
  }
  if (streaming)
    return launched(mbq::launch_decode_stream(*desc, packed, t, x, xb, perm, offsets, y, yb, lws,
                                              inline_u ? nullptr : u, inline_u ? 0 : ksu, b, rank,
                                              inline_u ? fz : nullptr, a, stream));
  if (!generic && t > 64 && mbq::prefill_mfma_supported(*desc, t, x, xb))
    return launched(mbq::launch_prefill_mfma(*desc, packed, t, x, xb, perm, offsets, y, yb, u, ksu, b,
                                             rank, opts->prefill_slots, stream));
  // the generic kernels: the side path is added to y afterwards
  if (t <= 64)
    st = launched(mbq::launch_decode(*desc, packed, t, x, xb, perm, offsets, y, yb, lws, stream));
  else
    st = launched(mbq::launch_prefill(*desc, packed, t, x, xb, perm, offsets, y, yb, stream));
  if (st != MBQ_OK || !lr) return st;
  return launched(mbq::launch_lowrank_update(t, desc->n, u, ksu, b, rank, y, yb, stream));
}

// The buffer of mbq_linear_static: file-scope device memory, one copy on every GPU the
// library runs on.  In host code `scratch` names a host-side stand-in, not a device
// address: its address on a device comes from hipGetSymbolAddress with that device
// current, resolved once per device and kept here; only that pointer reaches a kernel.
constexpr size_t kStaticScratchBytes = MBQ_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

mbq_status static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MBQ_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      if (std::getenv("MBQ_DEBUG")) std::fprintf(stderr, "libmbq: hipGetSymbolAddress failed: %s\n", hipGetErrorString(e));
      return MBQ_ERR_DEVICE;
    }
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return MBQ_OK;
}

}  // namespace

mbq_status mbq_linear_workspace(const mbq_desc* desc, int32_t t, mbq_dtype x_dtype,
                                size_t* bytes) {
  mbq_status st = check_desc(desc);
  if (st != MBQ_OK) return st;
  if (!bytes || !valid_dtype(x_dtype)) return MBQ_ERR_ARG;
  if (t < 0 || t > (1 << 24)) return MBQ_ERR_SHAPE;
  *bytes = linear_ws(*desc, t, x_dtype == MBQ_BF16, false);
  return MBQ_OK;
}

mbq_status mbq_linear(const mbq_desc* desc, const void* packed, int32_t t, const void* x,
                      mbq_dtype x_dtype, const int32_t* perm, const int32_t* offsets,
                      void* y, mbq_dtype y_dtype, void* workspace, size_t ws_bytes,
                      const mbq_opts* opts, hipStream_t stream) {
  return linear_impl(desc, packed, t, x, x_dtype, perm, offsets, nullptr, nullptr, 0, y, y_dtype,
                     workspace, ws_bytes, opts, stream);
}

mbq_status mbq_linear_static(const mbq_desc* desc, const void* packed, int32_t t, const void* x,
                             mbq_dtype x_dtype, const int32_t* perm, const int32_t* offsets,
                             void* y, mbq_dtype y_dtype, const mbq_opts* opts, hipStream_t stream) {
  mbq_status st = check_desc(desc);
  if (st != MBQ_OK) return st;
  if (!checked_opts(opts)) return MBQ_ERR_ARG;
  if (t < 0 || t > (1 << 24)) return MBQ_ERR_SHAPE;
  if (!valid_dtype(x_dtype) || !valid_dtype(y_dtype)) return MBQ_ERR_ARG;
  if (t > 0 && !linear_ptrs_ok(packed, x, perm, offsets, y)) return MBQ_ERR_ARG;  // before any device call
  const size_t need = t > 0 ? linear_ws(*desc, t, x_dtype == MBQ_BF16, false) : 0;
  if (need > kStaticScratchBytes) return MBQ_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    st = static_scratch(&ws);
    if (st != MBQ_OK) return st;
  }
  return linear_impl(desc, packed, t, x, x_dtype, perm, offsets, nullptr, nullptr, 0, y, y_dtype, ws,
                     need > 0 ? kStaticScratchBytes : 0, opts, stream);
}

mbq_status mbq_route_linear(const mbq_desc* desc, const void* packed, int32_t t, const void* x,
                            mbq_dtype x_dtype, const float* wr, float* logits, int32_t* budget,
                            int32_t* perm, int32_t* offsets, void* y, mbq_dtype y_dtype,
                            void* workspace, size_t ws_bytes, const mbq_opts* opts_in,
                            hipStream_t stream) {
  mbq_status st = check_desc(desc);
  if (st != MBQ_OK) return st;
  const mbq_opts* opts = checked_opts(opts_in);
  if (!opts) return MBQ_ERR_ARG;
  if (t < 0 || t > (1 << 24)) return MBQ_ERR_SHAPE;
  if (!valid_dtype(x_dtype) || !valid_dtype(y_dtype)) return MBQ_ERR_ARG;
  if (!offsets) return MBQ_ERR_ARG;
  if (t > 0 && (!packed || !x || !wr || !logits || !budget || !perm || !y)) return MBQ_ERR_ARG;
  if (t > 0 && x_dtype == MBQ_BF16 && opts->path != MBQ_PATH_GENERIC &&
      mbq::decode_route_supported(*desc, t)) {
    if (!aligned(packed, 256) || !aligned(x, 16) || !aligned(y, 16) || !aligned(logits, 4) ||
        !aligned(budget, 4) || !aligned(perm, 4) || !aligned(offsets, 4))
      return MBQ_ERR_ARG;
    if (workspace && !aligned(workspace, 16)) return MBQ_ERR_WORKSPACE;
    if (opts->decode_launches == 2 && ws_bytes < mbq::decode_route_workspace(*desc, t)) return MBQ_ERR_WORKSPACE;
    if (aligned(wr, 16))
      return launched(mbq::launch_decode_route(*desc, packed, t, x, wr, logits, budget, perm, offsets,
                                               y, y_dtype == MBQ_BF16, opts->decode_mul,
                                               opts->decode_launches, workspace, ws_bytes, stream));
  }
  st = mbq_route(t, desc->k, desc->slices, x, x_dtype, wr, logits, budget, perm, offsets, stream);
  if (st != MBQ_OK) return st;
  return mbq_linear(desc, packed, t, x, x_dtype, perm, offsets, y, y_dtype, workspace, ws_bytes, opts,
                    stream);
}

mbq_status mbq_route_linear_workspace(const mbq_desc* desc, int32_t t, mbq_dtype x_dtype, size_t* bytes) {
  mbq_status st = check_desc(desc);
  if (st != MBQ_OK) return st;
  if (!bytes || !valid_dtype(x_dtype)) return MBQ_ERR_ARG;
  if (t < 0 || t > (1 << 24)) return MBQ_ERR_SHAPE;
  const size_t lin = linear_ws(*desc, t, x_dtype == MBQ_BF16, false);
  *bytes = x_dtype == MBQ_BF16 ? std::max(lin, mbq::decode_route_workspace(*desc, t)) : lin;
  return MBQ_OK;
}

mbq_status mbq_route_prepare_workspace(const mbq_desc* desc, int32_t t, size_t* bytes) {
  mbq_status st = check_desc(desc);
  if (st != MBQ_OK) return st;
  if (!bytes) return MBQ_ERR_ARG;
  if (t < 0 || t > (1 << 24)) return MBQ_ERR_SHAPE;
  *bytes = mbq::decode_route_workspace(*desc, t);
  return MBQ_OK;
}

mbq_status mbq_route_prepare(const mbq_desc* desc, int32_t t, const void* x, const float* wr, void* prep,
                             size_t prep_bytes, hipStream_t stream) {
  mbq_status st = check_desc(desc);
  if (st != MBQ_OK) return st;
  if (t < 0 || t > (1 << 24)) return MBQ_ERR_SHAPE;
  if (t == 0) return MBQ_OK;
  if (!mbq::decode_prepared_supported(*desc, t)) return MBQ_ERR_UNSUPPORTED;
  if (!x || !wr || !aligned(x, 16) || !aligned(wr, 16)) return MBQ_ERR_ARG;
  if (!prep || !aligned(prep, 16) || prep_bytes < mbq::decode_route_workspace(*desc, t)) return MBQ_ERR_WORKSPACE;
  return launched(mbq::launch_decode_prepare(*desc, t, x, wr, prep, stream));
}

mbq_status mbq_route_linear_prepared(const mbq_desc* desc, const void* packed, int32_t t, const void* prep,
                                     size_t prep_bytes, float* logits, int32_t* budget, int32_t* perm,
                                     int32_t* offsets, void* y, mbq_dtype y_dtype, hipStream_t stream) {
  mbq_status st = check_desc(desc);
  if (st != MBQ_OK) return st;
  if (t < 0 || t > (1 << 24)) return MBQ_ERR_SHAPE;
  if (!valid_dtype(y_dtype) || !offsets || !aligned(offsets, 4)) return MBQ_ERR_ARG;
  if (t == 0) return MBQ_OK;
  if (!mbq::decode_prepared_supported(*desc, t)) return MBQ_ERR_UNSUPPORTED;
  if (!packed || !logits || !budget || !perm || !y) return MBQ_ERR_ARG;
  if (!aligned(packed, 256) || !aligned(y, 16) || !aligned(logits, 4) || !aligned(budget, 4) ||
      !aligned(perm, 4))
    return MBQ_ERR_ARG;
  if (!prep || !aligned(prep, 16) || prep_bytes < mbq::decode_route_workspace(*desc, t)) return MBQ_ERR_WORKSPACE;
  return launched(mbq::launch_decode_prepared(*desc, packed, t, prep, logits, budget, perm, offsets, y,
                                              y_dtype == MBQ_BF16, stream));
}

mbq_status mbq_linear_lowrank_workspace(const mbq_desc* desc, int32_t t, mbq_dtype x_dtype,
                                        int32_t rank, size_t* bytes) {
  mbq_status st = check_desc(desc);
  if (st != MBQ_OK) return st;
  if (!bytes || !valid_dtype(x_dtype)) return MBQ_ERR_ARG;
  if (t < 0 || t > (1 << 24)) return MBQ_ERR_SHAPE;
  if (!rank_ok(rank)) return MBQ_ERR_UNSUPPORTED;
  *bytes = t == 0 ? 0 : lr_state_bytes(t, rank) + u_bytes(t, desc->k, rank) + linear_ws(*desc, t, x_dtype == MBQ_BF16, true);
  return MBQ_OK;
}

mbq_status mbq_linear_lowrank(const mbq_desc* desc, const void* packed, int32_t t, const void* x,
                              mbq_dtype x_dtype, const int32_t* perm, const int32_t* offsets,
                              const uint16_t* a, const uint16_t* b, int32_t rank, void* y,
                              mbq_dtype y_dtype, void* workspace, size_t ws_bytes,
                              const mbq_opts* opts, hipStream_t stream) {
  if (!rank_ok(rank)) return MBQ_ERR_UNSUPPORTED;
  return linear_impl(desc, packed, t, x, x_dtype, perm, offsets, a, b, rank, y, y_dtype, workspace,
                     ws_bytes, opts, stream);
}

}  // extern "C"
