/*
 * mbq.h -- C ABI of the routed bit-sliced linear library (libmbq.so), gfx950 / MI355X.
 *
 * What it computes (MoBiQuant: Mixture-of-Bits Quantization for Token-Adaptive Elastic
 * LLMs; gist.science explainers, English page section 2 "Methodology", Japanese page
 * section 2 "Proposed method"):
 *   - MoBiSlice (section 2.A / 2.1): a weight matrix W [N x K] is decomposed into S
 *     2-bit slices by recursive residual quantization, R_0 = W, Q_j = Q(R_{j-1}),
 *     R_j = R_{j-1} - deq(Q_j); the first b slices summed give a 2b-bit weight
 *     W^(b) = sum_{j<=b} deq(Q_j), all from one stored copy.
 *   - MoBiRoute (section 2.B / 2.2): a per-token router decides how many slices b(t)
 *     each token activates.
 *   - The routed linear y_t = x_t . W^(b(t))^T, where a kernel fetches only the slices
 *     the tokens use (English page, section 3, "specialized kernel implementation").
 *
 * Readings of points the pages leave open (fixed here, identical in the CPU oracle):
 *   - Q is 2-bit asymmetric min/max round-to-nearest over groups of G consecutive inputs
 *     of one output row: scale = half((max - min) / 3), zero = half(min),
 *     code = clamp(rint((r - zero) / scale), 0, 3) (float32, IEEE divide, ties to even,
 *     code 0 when the stored scale is 0), deq = zero + code * scale rounded twice
 *     (float32 multiply, then float32 add; never fused).
 *   - The router is linear, no bias: logits = x . Wr, b(t) = 1 + first argmax.
 *   - The MLP router (mbq_route_mlp): scores = ReLU(x . W1^T + b1) . W2 + b2, one score
 *     per residual slice; the sigmoid gate passes slice j + 1 when sigmoid(score_j) >
 *     delta, evaluated as score_j > float32(logit(delta)); b(t) = 1 + the length of the
 *     leading run of passing slices.
 *   - Tokens are regrouped by a stable ascending sort on b(t).
 *
 * Conventions for every call:
 *   - All pointers except `mbq_desc*`, `bytes` and `out` are DEVICE pointers owned by the
 *     caller.  The library allocates nothing and keeps no global state (except
 *     mbq_linear_static's fixed device buffer, below): calls are re-entrant and
 *     thread-safe.
 *   - Every call only enqueues work on `stream` and never synchronizes the host.
 *   - Argument, shape and alignment checks happen before any launch; failures return a
 *     negative mbq_status and launch nothing.  A failed launch returns MBQ_ERR_DEVICE.
 *   - Alignment: the packed blob 256 bytes, x / y / workspace 16 bytes, others 4 bytes.
 *   - Supported: bits == 2, 1 <= slices <= 4, group in {32, 64, 128, 256}, K % group == 0,
 *     N >= 1, K >= group, T >= 0.  Groups of 32 inputs run on the generic kernels only
 *     (a lane's 16-input code words pair up into one group, which the streaming decode
 *     and the MFMA prefill tiles do not split); the other groups run on either.  With T == 0 nothing is launched except that
 *     mbq_route / mbq_regroup still write offsets; T-sized pointers may then be NULL.
 */
#ifndef MBQ_H
#define MBQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MBQ_ABI_VERSION 3

typedef enum {
  MBQ_OK = 0,
  MBQ_ERR_ARG = -1,          /* NULL or misaligned pointer, unknown dtype, NULL desc */
  MBQ_ERR_SHAPE = -2,        /* N, K, T out of range, K % group != 0, desc inconsistent */
  MBQ_ERR_RANGE = -3,        /* a value outside what the blob format can hold */
  MBQ_ERR_WORKSPACE = -4,    /* workspace NULL or smaller than mbq_linear_workspace() */
  MBQ_ERR_DEVICE = -5,       /* the HIP launch failed (hipGetLastError) */
  MBQ_ERR_UNSUPPORTED = -6,  /* group, slices, bits or ABI version not supported */
  /* range markers, never returned: they make every int32 value a valid mbq_status, so a
     caller's unknown code reaches mbq_status_str without undefined behaviour */
  MBQ_STATUS_MIN_ = INT32_MIN,
  MBQ_STATUS_MAX_ = INT32_MAX
} mbq_status;

/* Element types.  Any other int32 value is MBQ_ERR_ARG (the range markers make it a valid
   mbq_dtype, so the check itself is defined). */
typedef enum { MBQ_F32 = 0, MBQ_BF16 = 1, MBQ_DTYPE_MIN_ = INT32_MIN, MBQ_DTYPE_MAX_ = INT32_MAX } mbq_dtype;

/*
 * Kernel and tiling choices of the routed linear, for tests and tuning.  Every call that
 * takes `const mbq_opts* opts` accepts NULL for "every field 0" (automatic choices).  A
 * field outside its range is MBQ_ERR_ARG.  No choice changes what is computed beyond the
 * stated precision of the multiply it selects.
 */
typedef enum {
  MBQ_PATH_AUTO = 0,     /* the streaming decode (t <= 64) and the MFMA prefill (t > 64) where they apply */
  MBQ_PATH_GENERIC = 1,  /* the generic decode and prefill kernels (those that serve slices or
                            activations of 4 GiB and more) */
} mbq_path;

typedef enum {
  MBQ_MUL_AUTO = 0,      /* the plan's choice (see mbq_route_linear) */
  MBQ_MUL_BF16 = 1,      /* codes as bfloat16 (o + q) values, activations as they are: exact products */
  MBQ_MUL_FP8_FP4 = 2,   /* codes as e2m1, activations as an exact e4m3 hi + lo pair per 128 inputs */
} mbq_mul;

typedef struct {
  int32_t path;            /* mbq_path */
  int32_t decode_mul;      /* mbq_mul of the routed decode step (mbq_route_linear) */
  int32_t prefill_slots;   /* workgroups the MFMA prefill's tile plan assumes run at once
                              (0: the device's compute units); it decides which full tiles are
                              split in two, never the results */
  int32_t decode_launches; /* launches of the fp8 x fp4 decode step (mbq_route_linear): 0 the
                              plan's choice, 1 one, 2 two (operands prepared once, in the
                              workspace) */
} mbq_opts;

/*
 * Geometry of one packed weight (the "one checkpoint for every precision" of the
 * English page, section 3).  Filled by mbq_describe(); treat as read-only.
 *
 * Blob layout (slice-major, so a token that uses b slices reads only the first b):
 *   slice j (0-based) occupies bytes [j*slice_stride, (j+1)*slice_stride):
 *     codes  at +0:              row_blocks*k_tiles tiles of 1024 bytes; tile
 *                                (nb, kb) at (nb*k_tiles + kb)*1024; inside a tile,
 *                                lane l = 16*c + r owns 16 bytes at 16*l = four 32-bit
 *                                little-endian words; word i holds the 2-bit codes of
 *                                row 16*nb + r at inputs 256*kb + 64*i + 16*c + e,
 *                                e = 0..15; code e in bits [p, p+1] with
 *                                p = 16*(e & 1) + 2*(e >> 1) (even inputs in the low
 *                                half-word, odd inputs in the high half-word).
 *     params at +params_offset:  entry (nb, g, r) is 4 bytes at
 *                                ((nb*groups_padded + g)*16 + r)*4: half scale in
 *                                bits 0..15, half zero in bits 16..31.
 *   Rows >= n and inputs >= k are padding: code 0, params (0, 0).
 */
typedef struct {
  int32_t abi;            /* MBQ_ABI_VERSION */
  int32_t n, k;           /* output rows, inputs */
  int32_t group;          /* G: inputs per (scale, zero) group */
  int32_t slices;         /* S: 2-bit slices stored */
  int32_t bits;           /* bits per slice: 2 */
  int32_t row_blocks;     /* ceil(n / 16) */
  int32_t k_tiles;        /* ceil(k / 256) */
  int32_t groups_padded;  /* k_tiles * 256 / group */
  int32_t reserved;
  uint64_t codes_bytes;   /* per slice: row_blocks * k_tiles * 1024 */
  uint64_t params_bytes;  /* per slice: row_blocks * groups_padded * 64 */
  uint64_t params_offset; /* codes_bytes rounded up to 256 */
  uint64_t slice_stride;  /* params_offset + params_bytes rounded up to 256 */
  uint64_t total_bytes;   /* slices * slice_stride */
} mbq_desc;

/* Host only: validates the shape and fills *out.  Launches nothing. */
mbq_status mbq_describe(int32_t n, int32_t k, int32_t group, int32_t slices, mbq_desc* out);

/*
 * MoBiSlice pack (English page section 2.A; Japanese page section 2.1).
 *   w:          [n x k] row-major weights, float32 or bfloat16 (w_dtype).
 *   packed:     desc->total_bytes, 256-byte aligned; fully overwritten (padding too).
 *   dev_status: nullable int32; the kernel ORs in bit 0 if W holds a non-finite value
 *               and bit 1 if a scale or zero overflowed half.  The caller clears it
 *               before the call and reads it after synchronizing.  With a nonzero
 *               status the blob contents are unspecified.
 */
mbq_status mbq_pack(const mbq_desc* desc, const void* w, mbq_dtype w_dtype, void* packed,
                    int32_t* dev_status, hipStream_t stream);

/*
 * Bit-plane pack: the other reading of the English page's "MSB slice plus residual bit
 * slices" (section 2.A; Japanese page section 2.1).  Each weight gets one uniform 2S-bit
 * min/max code per group (4^S levels, step = half((max - min) / (4^S - 1)), zero =
 * half(min), code = clamp(rint((w - zero) / step), 0, 4^S - 1), float32 as in mbq_pack);
 * slice j (1-based) stores the code's j-th 2-bit plane from the top, with scale
 * half(step * 4^(S-j)) and zero half(zero + c_1) for j = 1, half(c_j - c_(j-1)) after,
 * c_b = step * (4^(S-b) - 1) / 2, so that the linear kernels' prefix sum over b slices is
 * the b-plane value centred over the dropped planes.  Same blob layout, arguments and
 * status bits as mbq_pack; the routed linear is unchanged.
 */
mbq_status mbq_pack_bitplane(const mbq_desc* desc, const void* w, mbq_dtype w_dtype, void* packed,
                             int32_t* dev_status, hipStream_t stream);

/*
 * MoBiSlice pack of a row range: W_part [rows x k] becomes rows row0 .. row0 + rows - 1 of
 * the blob described by desc (desc->n rows in all).  Quantization groups lie within one
 * row, so the codes and params of those rows are exactly what mbq_pack of the whole
 * weight would write.  This lets weights that read the same activations (q/k/v, gate/up)
 * share one blob and one routed linear launch (English page section 4: the kernels'
 * efficiency at decoder-layer sizes).
 *   row0:   multiple of 16; rows >= 1; row0 + rows <= desc->n; rows is a multiple of 16
 *           unless the part ends the blob (MBQ_ERR_SHAPE otherwise).
 *   The blob is fully defined once parts cover rows 0 .. desc->n - 1; the part holding
 *   the last row also writes the blob's trailing alignment bytes.  Parts write disjoint
 *   bytes and may run concurrently.  w, dev_status: as in mbq_pack.
 */
mbq_status mbq_pack_rows(const mbq_desc* desc, int32_t row0, int32_t rows, const void* w,
                         mbq_dtype w_dtype, void* packed, int32_t* dev_status, hipStream_t stream);

/*
 * MoBiRoute (English page section 2.B; Japanese page section 2.2), linear-argmax form.
 *   x:       [t x k] tokens (float32 or bfloat16), or NULL to route from the caller's
 *            `logits` instead ("logits-in" mode).
 *   wr:      [k x s] float32 router weights (ignored when x is NULL).
 *   logits:  [t x s] float32; written (x != NULL) or read (x == NULL).
 *   budget:  [t] int32 out, b(t) = 1 + first index of the largest logit.
 *   perm:    [t] int32 out, stable ascending order of tokens by budget.
 *   offsets: [s + 1] int32 out, offsets[i] = #tokens with budget <= i.
 * NaN logits are outside the contract.  1 <= s <= 4, t <= 1<<24.
 */
mbq_status mbq_route(int32_t t, int32_t k, int32_t s, const void* x, mbq_dtype x_dtype,
                     const float* wr, float* logits, int32_t* budget, int32_t* perm,
                     int32_t* offsets, hipStream_t stream);

/*
 * Regroup tokens whose budgets are given (forced mixes): the stable counting sort of
 * mbq_route without the router.  budget values must lie in [1, s].
 */
mbq_status mbq_regroup(int32_t t, int32_t s, const int32_t* budget, int32_t* perm,
                       int32_t* offsets, hipStream_t stream);

/* Host only: bytes of device workspace mbq_route_mlp needs for t tokens of k inputs and
 * `hidden` hidden units: float32 partial hidden sums, c * t * hidden * 4 bytes, where c
 * is the number of K chunks the launch uses (c <= 64, chosen from t, k and hidden only),
 * then, for t <= 64, 256 bytes of per-token budget words through which the gate's
 * workgroups hand their budgets to the one that regroups.  0 when t == 0. */
mbq_status mbq_route_mlp_workspace(int32_t t, int32_t k, int32_t hidden, size_t* bytes);

/*
 * MoBiRoute in the pages' own form (English page section 2.B; Japanese page section 2.2):
 * a 2-layer MLP scores each token once per residual slice, and a sigmoid gate with
 * threshold delta turns the scores into a binary slice mask (a larger delta activates
 * fewer slices, so delta sets the average bit width at run time).
 *   x:       [t x k] tokens (float32 or bfloat16), or NULL to gate the caller's `scores`
 *            instead ("scores-in" mode; w1, b1, w2, b2 and workspace are then ignored).
 *   w1:      [hidden x k] bfloat16 bit patterns, row-major (row u = input weights of
 *            hidden unit u).  float32 x is multiplied as a bfloat16 hi + lo pair.
 *   b1:      [hidden] float32, 16-byte aligned.
 *   w2:      [hidden x (s - 1)] float32, row-major.   b2: [s - 1] float32.
 *   delta:   gate threshold; delta <= 0 passes every slice, delta >= 1 none; NaN is
 *            MBQ_ERR_RANGE.
 *   scores:  [t x (s - 1)] float32; written (x != NULL) or read (x == NULL); may be NULL
 *            when s == 1.  scores = ReLU(x . W1^T + b1) . W2 + b2, float32 accumulation
 *            in a fixed order (identical from run to run).
 *   budget:  [t] int32 out, b(t) = 1 + #leading j with scores[t][j] > float32(logit(delta)).
 *   perm, offsets: as in mbq_route.
 *   workspace: at least mbq_route_mlp_workspace() bytes, 16-byte aligned (may be NULL when
 *            that is 0 or in scores-in mode); overwritten.
 * hidden must be a multiple of 64 in [64, 4096]; t * k * sizeof(x) and hidden * k * 2
 * must stay below 2^31 bytes.  NaN scores are outside the contract.  1 <= s <= 4.
 */
mbq_status mbq_route_mlp(int32_t t, int32_t k, int32_t s, int32_t hidden, const void* x,
                         mbq_dtype x_dtype, const uint16_t* w1, const float* b1,
                         const float* w2, const float* b2, double delta, float* scores,
                         int32_t* budget, int32_t* perm, int32_t* offsets, void* workspace,
                         size_t ws_bytes, hipStream_t stream);

/* Host only: bytes of device workspace mbq_linear needs for t tokens (0 when none).
 * Decode (1 <= t <= 64) over more k tiles of 256 inputs than one workgroup holds (8 waves
 * of 1 or 2 tiles each: 2 when the group / slices / x dtype variant fits its registers,
 * 1 when t > 32 and two 16-token blocks share each workgroup) splits K into c equal
 * chunks and needs c * t * n * 4 bytes of float32 partials; prefill needs none.  The
 * size depends only on desc, t and x_dtype. */
mbq_status mbq_linear_workspace(const mbq_desc* desc, int32_t t, mbq_dtype x_dtype,
                                size_t* bytes);

/*
 * Routed linear y_t = x_t . (sum_{j <= b(t)} deq(Q_j))^T (English page sections 2.A and
 * 3: each token reconstructs its own precision from the shared slices; slices no token
 * uses are never read).
 *   packed:  the blob written by mbq_pack for `desc`.
 *   x:       [t x k] row-major, float32 or bfloat16, original token order.
 *   perm, offsets: as produced by mbq_route / mbq_regroup for these t tokens
 *            (offsets has desc->slices + 1 entries; the token at sorted position i has
 *            budget b with offsets[b-1] <= i < offsets[b]).
 *   y:       [t x n] row-major, float32 or bfloat16, original token order; every element
 *            is written.  Accumulation is float32; bfloat16 output is rounded once.
 *   workspace: at least mbq_linear_workspace() bytes (16-byte aligned; may be NULL when
 *            that is 0); contents are scratch, overwritten by every call that uses it, so
 *            calls that overlap in time must not share one.
 * Decode (t <= 64) runs a streaming kernel that reads each needed slice once (a slice no
 * token uses is not read at all), in 16-token blocks, with K split into chunks whose
 * partials a second small kernel sums in a fixed order when K is long; prefill
 * (t > 64) runs an MFMA GEMM over tiles of one budget group each: the summed slices are
 * dequantized to bfloat16 MFMA operands once per 256-token tile and shared between the
 * two waves of a SIMD through LDS.  Full tiles past the first round of workgroups (one
 * per CU) are split into 128-token tiles when that lets the second round fit
 * (opts->prefill_slots sets the workgroup count that rule assumes).  Rows whose perm entry
 * is outside [0, t) are not written; offsets outside [0, t] are clamped (no access outside
 * x, y, perm).
 *   opts:    NULL or kernel choices (mbq_opts); opts->decode_mul is ignored here.
 */
mbq_status mbq_linear(const mbq_desc* desc, const void* packed, int32_t t, const void* x,
                      mbq_dtype x_dtype, const int32_t* perm, const int32_t* offsets,
                      void* y, mbq_dtype y_dtype, void* workspace, size_t ws_bytes,
                      const mbq_opts* opts, hipStream_t stream);

/*
 * mbq_linear for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The same routed linear
 * (same kernels, same results), with the split-K partials of the streaming decode kept in
 * a buffer of MBQ_STATIC_SCRATCH_BYTES that the library holds in the device memory of every
 * GPU it runs on (reserved with the library's code, held until the process ends) instead
 * of a caller workspace.  The call allocates nothing and frees nothing.
 *   Arguments as in mbq_linear, without workspace and ws_bytes.
 *   Returns MBQ_ERR_WORKSPACE, launching nothing, when mbq_linear_workspace() for these
 *   arguments exceeds MBQ_STATIC_SCRATCH_BYTES (e.g. 64 tokens of a 18944 x 13824 weight).
 *   The first call on each device resolves that device's buffer address
 *   (hipGetSymbolAddress, with the device current); MBQ_ERR_DEVICE if that fails.
 *   All calls on one GPU share its one buffer, which keeps the last call's partials:
 *   calls that overlap in time on the same GPU (two streams, or two host threads) race,
 *   and the caller must serialize them.
 */
#define MBQ_STATIC_SCRATCH_BYTES (16u << 20)
mbq_status mbq_linear_static(const mbq_desc* desc, const void* packed, int32_t t, const void* x,
                             mbq_dtype x_dtype, const int32_t* perm, const int32_t* offsets,
                             void* y, mbq_dtype y_dtype, const mbq_opts* opts, hipStream_t stream);

/*
 * The routed fp8 x fp4 decode step in two calls (English page sections 2.A, 2.B and 3; the
 * same results as mbq_route_linear with that multiply): mbq_route_prepare turns t <= 16
 * bfloat16 tokens into what every workgroup of the streaming kernel needs -- the
 * activations as exact e4m3 hi + lo pairs with one power-of-two scale per token and 128
 * inputs, their per-group sums, and per k tile of 256 inputs the partial router logits
 * (Wr as three exact bfloat16 planes, float32 sums) -- and mbq_route_linear_prepared
 * completes the routing (partial logits summed in tile order, first argmax, stable
 * regroup; writes logits, budget, perm, offsets) and runs the routed linear on them.  One
 * prepared buffer serves every weight with the same desc->k, group and slices.
 *   prep, prep_bytes: device buffer of at least mbq_route_prepare_workspace() bytes,
 *                     16-byte aligned (MBQ_ERR_WORKSPACE otherwise); written by prepare,
 *                     read by prepared.
 *   x: [t x desc->k] bfloat16, wr: [desc->k x desc->slices] float32, both 16-byte aligned.
 *   Other arguments as in mbq_route_linear.  MBQ_ERR_UNSUPPORTED where mbq_route_linear
 *   would not run the step as one kernel (t > 16, K beyond one workgroup) or for blobs of
 *   one slice; mbq_route_prepare_workspace() returns 0 there.
 */
mbq_status mbq_route_prepare_workspace(const mbq_desc* desc, int32_t t, size_t* bytes);
mbq_status mbq_route_prepare(const mbq_desc* desc, int32_t t, const void* x, const float* wr, void* prep,
                             size_t prep_bytes, hipStream_t stream);
mbq_status mbq_route_linear_prepared(const mbq_desc* desc, const void* packed, int32_t t, const void* prep,
                                     size_t prep_bytes, float* logits, int32_t* budget, int32_t* perm,
                                     int32_t* offsets, void* y, mbq_dtype y_dtype, hipStream_t stream);

/* Host only: bytes of device workspace mbq_route_linear can use for t tokens: the
 * prepared operands of its two-launch fp8 x fp4 step (see there), or the routed linear's
 * (mbq_linear_workspace), whichever is larger.  Depends only on desc, t and x_dtype. */
mbq_status mbq_route_linear_workspace(const mbq_desc* desc, int32_t t, mbq_dtype x_dtype,
                                      size_t* bytes);

/*
 * One decode step in one call: MoBiRoute (linear-argmax form) and the routed linear
 * (English page sections 2.A, 2.B and 3).  Results are those of mbq_route(t, desc->k,
 * desc->slices, x, x_dtype, wr, logits, budget, perm, offsets) followed by
 * mbq_linear(desc, packed, t, x, x_dtype, perm, offsets, y, ...), except that the logits
 * are summed in another order (they may differ from mbq_route's in the last bits; budget,
 * perm and offsets are exactly the argmax and stable regroup of the logits written here).
 *   wr, logits, budget, perm, offsets: as in mbq_route; all written.
 *   y, y_dtype, workspace, ws_bytes: as in mbq_linear (size from mbq_linear_workspace).
 * With bfloat16 x, 1 <= t <= 16, K within one workgroup of the streaming decode kernel
 * (at most 16 k tiles of 256 where a wave holds two, 8 where it holds one) and wr 16-byte
 * aligned, that kernel routes the batch itself: every workgroup multiplies the
 * activations it already holds by Wr (fixed summation order, so all of them reach the
 * same budgets) and workgroup 0 writes the routing outputs -- one launch instead of
 * three.  Where each workgroup streams 4 or more row blocks of 16 outputs over 2 or more
 * slices, that kernel multiplies on the fp8 x fp4 matrix instruction instead of bf16:
 * codes enter exactly, the activations as an exact e4m3 pair per 128 inputs, and the
 * instruction's own sum adds an error of about 1e-5 of the sum of |products| (y stays
 * within 1e-3 per token of the bf16 multiply); opts->decode_mul forces either multiply
 * (a blob of one slice always takes the bf16 multiply).
 * Otherwise (or with opts->path == MBQ_PATH_GENERIC) the two calls run in sequence.
 * Errors as in the two calls.
 */
mbq_status mbq_route_linear(const mbq_desc* desc, const void* packed, int32_t t, const void* x,
                            mbq_dtype x_dtype, const float* wr, float* logits, int32_t* budget,
                            int32_t* perm, int32_t* offsets, void* y, mbq_dtype y_dtype,
                            void* workspace, size_t ws_bytes, const mbq_opts* opts,
                            hipStream_t stream);

/* Host only: bytes of device workspace mbq_linear_lowrank needs: the side path's call
 * state (256 bytes, 512 check-in lines of 128 bytes, then u of every 16-token block as
 * 8-byte pairs: 16 ceil(t/16) rank x 8 bytes rounded up to 256), u as c float32
 * partials over chunks of K ([c x t x rank],
 * c <= 8 chosen from t and k; rounded up to 256 bytes), then the routed linear's split-K
 * partials under the side path's plan (one 16-token block per workgroup).  0 when
 * t == 0. */
mbq_status mbq_linear_lowrank_workspace(const mbq_desc* desc, int32_t t, mbq_dtype x_dtype,
                                        int32_t rank, size_t* bytes);

/*
 * Routed linear with a low-rank side path: W ~ W^(b) + B A (TTQ Japanese page, section 2:
 * a quantized weight plus rank-r factors kept beside it; section 4: rank 16), so
 *   y_t = x_t . W^(b(t))^T + (x_t . A^T) . B^T
 * with one (A, B) pair for every token whatever its budget.
 *   a:     [rank x k] bfloat16 bit patterns, row-major, 16-byte aligned.
 *   b:     [n x rank] bfloat16 bit patterns, row-major, 16-byte aligned.
 *   rank:  a multiple of 8 in [8, 32] (MBQ_ERR_UNSUPPORTED otherwise).
 *   workspace: at least mbq_linear_lowrank_workspace() bytes, 16-byte aligned.  Its
 *           front part carries state from one call to the next: fill the whole workspace
 *           with zeros before its first call and write nothing into it between calls
 *           (every call leaves that state ready for the next; calls on one workspace must
 *           not overlap).  A workspace at least as large serves every t and shape.
 *   Other arguments (opts too) as in mbq_linear.
 * u = x . A^T (float32 accumulation over k; float32 x as a bf16 hi + lo pair) is added
 * as u . B^T to the linear kernels' float32 accumulators before the one rounding to y (u
 * enters their MFMAs as a bf16 hi + lo pair).  The streaming decode (t <= 64, K within
 * one workgroup) computes u inside its own launch: workgroup 0 of every 16-token block
 * multiplies the activations by A and publishes u in the workspace with this call's tag;
 * the other workgroups stream the weight and pick u up for their first row block one row
 * block later.  Elsewhere u is computed by a launch of its own first.  Kernels without
 * the fusion (the generic decode and prefill) add u . B^T to y afterwards; bfloat16 y is
 * then rounded twice.
 */
mbq_status mbq_linear_lowrank(const mbq_desc* desc, const void* packed, int32_t t, const void* x,
                              mbq_dtype x_dtype, const int32_t* perm, const int32_t* offsets,
                              const uint16_t* a, const uint16_t* b, int32_t rank, void* y,
                              mbq_dtype y_dtype, void* workspace, size_t ws_bytes,
                              const mbq_opts* opts, hipStream_t stream);

/* Static string for a status code. */
const char* mbq_status_str(mbq_status status);

/* MBQ_ABI_VERSION of the loaded library. */
int32_t mbq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MBQ_H */
