"""CPU oracle for the routed bit-sliced linear (MoBiQuant-style elastic weight quantization).

TEST INFRASTRUCTURE ONLY.  This module is a plain, slow, deliberately obvious numpy
implementation of what the hot path computes.  It exists so that tests, the smoke check
and the CPU baseline leg of the benchmark can compare the HIP library against it.  No
product code path may import, call or execute anything under ``oracle/``; the HIP library
shares no code, constants or helpers with it.

Sources (the pages; cited by title and section):
  * "MoBiQuant: Mixture-of-Bits Quantization for Token-Adaptive Elastic LLMs",
    gist.science explainer in English, section 2.A "MoBiSlice: Many-in-One Recursive
    Residual Quantization" (the residual recursion and the prefix-sum reconstruction),
    section 2.B "MoBiRoute: Token-Aware Routing" (a router scores each token and decides
    how many residual slices it activates), section 3 (kernels fetch only the bit slices
    a token uses).
  * The same paper's Japanese explainer (gist.science/ja), section 2.1 MoBiSlice
    (R_1 = W, W_e = Q(R_e), R_{e+1} = R_e - W_e, and W^(b) = sum of the slices) and
    section 2.2 MoBiRoute.

Readings where the pages leave a step open:
  * Q is 2-bit asymmetric min/max round-to-nearest per group of G consecutive inputs of
    one output row: scale = (max - min) / 3, zero = min, both stored as IEEE half, codes
    = clamp(rint((r - zero) / scale), 0, 3) computed with the *stored* (rounded) params,
    dequantized value zero + code * scale.  The pages only write "Q(R_e)".
  * Pack arithmetic is float32 with every operation rounded on its own (no fused
    multiply-add), rint rounds half to even, a zero stored scale gives code 0, and a
    group minimum of -0 is stored as +0 (the pages say nothing about signed zeros).
  * The router is linear without bias; a token's slice count is 1 + the first index of
    the largest logit.  (The pages' own router is a 2-layer MLP with a threshold.)
  * The pages' MLP router, as built here: hidden = ReLU(x . W1^T + b1) (W1 [H, K]),
    scores = hidden . W2 + b2, one score per residual slice (S - 1 of them; the base
    slice is always used).  At inference the sigmoid gate passes a slice when
    sigmoid(score) > delta, which is evaluated exactly as score > theta with
    theta = logit(delta) rounded to float32 (delta <= 0 passes all, delta >= 1 none).
    Residual slices refine each other, so a token uses the leading run of passing
    slices: b = 1 + its length.  The pages name neither the activation nor the hidden
    width; ReLU is the plainest reading.
  * The low-rank side path of the TTQ explainer (section 2: W ~ Wq + BA, with the
    quantized part adjusted and the rank-r factors kept beside it; section 4: r = 16):
    here Wq is the token's MoBiSlice reconstruction W^(b), and B [N, r], A [r, K] are one
    pair shared by every token whatever its b, so y_t = x_t . W^(b(t))^T + (x_t . A^T) . B^T.
  * The bit-plane reading of the "MSB slice plus residual slices" wording (English
    explainer section 2.A, Japanese section 2.1): one uniform 2S-bit min/max code per
    weight (4^S levels, step = span / (4^S - 1), rounded to half, zero = half(min)), slice
    j holding its j-th 2-bit plane from the top.  The slice params are chosen so that the
    same prefix sum the kernels compute gives the b-plane value centred over the dropped
    planes: scale_j = step * 4^(S-j), zero_1 = min + c_1, zero_j = c_j - c_(j-1) with
    c_b = step * (4^(S-b) - 1) / 2 (each rounded to half).
  * Regrouping is a stable sort of tokens by ascending slice count.
  * Dot products and reconstruction are exact in float64 on the stored codes and params.

Parity pins: every public function here is pinned by tests in ``tests/test_oracle.py``
against brute force, closed forms, invariants and hand-worked fixtures; none is
"parity unpinned".
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
F16 = np.float16


# ----------------------------------------------------------------------------------------
# MoBiSlice: one 2-bit asymmetric round-to-nearest slice of a residual
# (MoBiQuant explainer, section 2.A; the quantizer Q itself is the reading above)
# ----------------------------------------------------------------------------------------
def quantize_slice(R: np.ndarray, group: int):
    """Quantize residual R (float32, [N, K]) with one 2-bit slice.

    Returns (codes uint8 [N, K], scale float16 [N, K/G], zero float16 [N, K/G],
    deq float32 [N, K], next_residual float32 [N, K], flags) where flags bit 1 is set if a
    stored scale or zero overflowed half precision.
    """
    R = np.asarray(R, dtype=F32)
    N, K = R.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    Rg = R.reshape(N, K // group, group)
    lo = Rg.min(axis=2)                       # exact
    hi = Rg.max(axis=2)                       # exact
    lo = (lo + F32(0.0)).astype(F32)          # a signed-zero minimum is stored as +0
    with np.errstate(over="ignore", invalid="ignore"):
        span = (hi - lo).astype(F32)          # one float32 rounding
        step32 = (span / F32(3.0)).astype(F32)  # one float32 rounding (IEEE divide)
        scale = step32.astype(F16)            # round to nearest even, subnormals kept
        zero = lo.astype(F16)
    flags = 0
    if not (np.all(np.isfinite(scale)) and np.all(np.isfinite(zero))):
        flags |= 2
    sf = scale.astype(F32)[:, :, None]
    zf = zero.astype(F32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        t = (Rg - zf).astype(F32)             # float32 subtract
        u = (t / sf).astype(F32)              # float32 divide
        q = np.clip(np.rint(u), 0.0, 3.0)     # half-to-even, then clamp
    q = np.where(sf == 0.0, 0.0, q)           # degenerate group: every code is 0
    q = q.astype(np.uint8)
    with np.errstate(invalid="ignore", over="ignore"):   # only when a param overflowed
        prod = (q.astype(F32) * sf).astype(F32)   # rounded multiply ...
        deq = (zf + prod).astype(F32)             # ... then rounded add (no FMA)
        nxt = (Rg - deq).astype(F32)
    return (q.reshape(N, K), scale, zero, deq.reshape(N, K), nxt.reshape(N, K), flags)


def pack(W: np.ndarray, group: int, slices: int):
    """MoBiSlice recursion: R_0 = W, Q_j = RTN2(R_{j-1}), R_j = R_{j-1} - deq(Q_j).

    W must be finite float32 (bfloat16 inputs are passed as their exact float32 values).
    Returns a dict with codes uint8 [S, N, K], scale/zero float16 [S, N, K/G], the float32
    residual after every slice (residuals [S+1, N, K], residuals[0] == W) and the OR of
    the per-slice overflow flags (bit 0 = non-finite W, bit 1 = half overflow).
    """
    W = np.asarray(W, dtype=F32)
    flags = 0
    if not np.all(np.isfinite(W)):
        flags |= 1
    N, K = W.shape
    codes = np.zeros((slices, N, K), np.uint8)
    scale = np.zeros((slices, N, K // group), F16)
    zero = np.zeros((slices, N, K // group), F16)
    residuals = np.zeros((slices + 1, N, K), F32)
    residuals[0] = W
    R = W
    for j in range(slices):
        q, s, z, _deq, R, f = quantize_slice(R, group)
        codes[j], scale[j], zero[j], residuals[j + 1] = q, s, z, R
        flags |= f
    return {"codes": codes, "scale": scale, "zero": zero, "residuals": residuals,
            "flags": flags, "group": group}


def pack_bitplane(W: np.ndarray, group: int, slices: int):
    """Bit-plane slices: planes of one uniform 2S-bit code per weight (see the reading
    above).  Same output layout as pack(): codes uint8 [S, N, K] (plane values 0..3),
    scale/zero float16 [S, N, K/G], flags; plus the full codes q [N, K] (uint16)."""
    W = np.asarray(W, dtype=F32)
    flags = 0 if np.all(np.isfinite(W)) else 1
    N, K = W.shape
    S = slices
    levels = 4 ** S - 1
    Wg = W.reshape(N, K // group, group)
    lo = (Wg.min(axis=2) + F32(0.0)).astype(F32)   # a signed-zero minimum is stored as +0
    hi = Wg.max(axis=2)
    with np.errstate(over="ignore", invalid="ignore"):
        span = (hi - lo).astype(F32)
        step = (span / F32(levels)).astype(F32).astype(F16)
        zero_h = lo.astype(F16)
    sf = step.astype(F32)
    zf = zero_h.astype(F32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        u = ((Wg - zf[:, :, None]).astype(F32) / sf[:, :, None]).astype(F32)
        q = np.clip(np.rint(u), 0.0, float(levels))
    q = np.where(sf[:, :, None] == 0.0, 0.0, q).astype(np.uint16)
    codes = np.zeros((S, N, K), np.uint8)
    scale = np.zeros((S, N, K // group), F16)
    zero = np.zeros((S, N, K // group), F16)
    with np.errstate(over="ignore", invalid="ignore"):
        c = [(sf * F32((4 ** (S - b) - 1) / 2)).astype(F32) for b in range(1, S + 1)]
        for j in range(1, S + 1):
            codes[j - 1] = ((q >> (2 * (S - j))) & 3).reshape(N, K).astype(np.uint8)
            scale[j - 1] = (sf * F32(4 ** (S - j))).astype(F32).astype(F16)
            z = (zf + c[0]) if j == 1 else (c[j - 1] - c[j - 2])
            zero[j - 1] = z.astype(F32).astype(F16)
    if not (np.all(np.isfinite(scale)) and np.all(np.isfinite(zero))):
        flags |= 2
    return {"codes": codes, "scale": scale, "zero": zero, "flags": flags, "group": group,
            "q": q.reshape(N, K), "step": step, "lo": zero_h}


# ----------------------------------------------------------------------------------------
# Elastic reconstruction W^(b) = sum_{j<=b} deq(Q_j), exact in float64
# (MoBiQuant explainer, section 2.A "Elasticity"; Japanese explainer section 2.1)
# ----------------------------------------------------------------------------------------
def dequant_slices(codes, scale, zero, group: int) -> np.ndarray:
    """Exact float64 dequantized slices DEQ_j[n, k] = zero_j[n, g] + code_j[n, k] * scale_j[n, g]."""
    S, N, K = codes.shape
    s = np.repeat(scale.astype(np.float64), group, axis=2)
    z = np.repeat(zero.astype(np.float64), group, axis=2)
    return z + codes.astype(np.float64) * s


def reconstruct(deq: np.ndarray, b: int) -> np.ndarray:
    """W^(b): the sum of the first b dequantized slices (float64)."""
    return deq[:b].sum(axis=0)


# ----------------------------------------------------------------------------------------
# MoBiRoute (MoBiQuant explainer, section 2.B): score each token, pick its slice count
# ----------------------------------------------------------------------------------------
def router_logits(X: np.ndarray, Wr: np.ndarray) -> np.ndarray:
    """Reference logits L = X . Wr in float64 (X [T, K], Wr [K, S])."""
    return np.asarray(X, np.float64) @ np.asarray(Wr, np.float64)


def route_from_logits(L: np.ndarray) -> np.ndarray:
    """b(t) = 1 + the first index holding the largest logit of token t (int32 [T]).

    Written as an explicit scan that replaces the running best only on a strictly larger
    value, which is what makes the lowest index win a tie.
    """
    L = np.asarray(L)
    T, S = L.shape
    out = np.empty(T, np.int32)
    for t in range(T):
        best, arg = L[t, 0], 0
        for j in range(1, S):
            if L[t, j] > best:
                best, arg = L[t, j], j
        out[t] = arg + 1
    return out


def regroup(budget: np.ndarray, slices: int):
    """Stable sort of tokens by ascending slice count.

    perm[i] = original index of the i-th token in sorted order; offsets[i] = number of
    tokens with budget <= i (offsets[0] = 0, offsets[S] = T).
    """
    budget = np.asarray(budget)
    perm = np.argsort(budget, kind="stable").astype(np.int32)
    offsets = np.zeros(slices + 1, np.int32)
    for i in range(1, slices + 1):
        offsets[i] = int(np.count_nonzero(budget <= i))
    return perm, offsets


# ----------------------------------------------------------------------------------------
# MoBiRoute as the pages describe it (English explainer section 2.B, Japanese section 2.2):
# a 2-layer MLP scores each token per residual slice; a sigmoid gate with threshold delta
# turns the scores into a binary mask at inference, and raising delta activates fewer slices
# ----------------------------------------------------------------------------------------
def mlp_router_scores(X, W1, b1, W2, b2) -> np.ndarray:
    """scores [T, S-1] = ReLU(X . W1^T + b1) . W2 + b2 in float64.

    X [T, K], W1 [H, K] (one row of input weights per hidden unit), b1 [H], W2 [H, S-1],
    b2 [S-1].
    """
    X, W1, b1, W2, b2 = (np.asarray(a, np.float64) for a in (X, W1, b1, W2, b2))
    hidden = np.maximum(X @ W1.T + b1, 0.0)
    return hidden @ W2 + b2


def gate_threshold(delta: float) -> np.float32:
    """theta such that sigmoid(s) > delta  <=>  s > theta: logit(delta) rounded to float32.

    sigmoid is increasing, so sigmoid(s) > delta exactly when s > log(delta / (1 - delta)).
    """
    if delta <= 0.0:
        return np.float32(-np.inf)
    if delta >= 1.0:
        return np.float32(np.inf)
    return np.float32(np.log(delta) - np.log1p(-delta))


def budgets_from_scores(scores, theta) -> np.ndarray:
    """b(t) = 1 + the number of leading residual slices whose score exceeds theta (int32)."""
    scores = np.asarray(scores)
    T, R = scores.shape
    out = np.empty(T, np.int32)
    for t in range(T):
        b = 1
        for j in range(R):
            if scores[t, j] > theta:
                b += 1
            else:
                break
        out[t] = b
    return out


def average_bits(budget, bits_per_slice: int = 2) -> float:
    """Average weight bit width over the tokens: bits_per_slice * mean(b)."""
    return float(bits_per_slice * np.mean(np.asarray(budget, np.float64)))


# ----------------------------------------------------------------------------------------
# Routed linear y_t = x_t . (sum_{j<=b(t)} deq(Q_j))^T in float64
# (MoBiQuant explainer, sections 2.A-2.B and 3: each token uses only its own slices)
# ----------------------------------------------------------------------------------------
def linear(X: np.ndarray, deq: np.ndarray, budget: np.ndarray) -> np.ndarray:
    """Y [T, N] in float64, original token order."""
    X = np.asarray(X, np.float64)
    budget = np.asarray(budget)
    T = X.shape[0]
    N = deq.shape[1]
    Y = np.zeros((T, N), np.float64)
    for b in range(1, deq.shape[0] + 1):
        idx = np.nonzero(budget == b)[0]
        if idx.size:
            Y[idx] = X[idx] @ reconstruct(deq, b).T
    return Y


def lowrank_term(X, A, B) -> np.ndarray:
    """The rank-r side path (TTQ explainer, section 2): (X . A^T) . B^T in float64, [T, N]."""
    X, A, B = (np.asarray(a, np.float64) for a in (X, A, B))
    return (X @ A.T) @ B.T


def linear_lowrank(X, deq, budget, A, B) -> np.ndarray:
    """Routed linear plus the side path: y_t = x_t . W^(b(t))^T + (x_t . A^T) . B^T."""
    return linear(X, deq, budget) + lowrank_term(X, A, B)


# ----------------------------------------------------------------------------------------
# The packed blob: slice-major storage so that fewer slices read fewer bytes
# (MoBiQuant explainer, section 3: kernels avoid an all-or-nothing fetch).
# This is a storage format; both sides implement it independently from this description:
#   * Row blocks of 16 rows (NB = ceil(N/16)), k tiles of 256 inputs (KB = ceil(K/256)),
#     NG = 256*KB/G groups per row (groups past K are padding).
#   * Slice j occupies bytes [j*slice_stride, (j+1)*slice_stride): its codes section
#     (NB*KB*1024 bytes) then, at the next 256-byte boundary, its params section
#     (NB*NG*64 bytes).  slice_stride = align256(codes) + align256(params).
#   * Codes: tile (nb, kb) is 1024 bytes at (nb*KB + kb)*1024; inside it, lane
#     l = 16*c + r (r = row in block, c = 0..3) owns 16 bytes at 16*l: four little-endian
#     32-bit words, word i holding the 16 codes of row 16*nb + r at inputs
#     k = 256*kb + 64*i + 16*c + e, e = 0..15; code e sits in bits p..p+1 with
#     p = 16*(e % 2) + 2*(e // 2): even inputs fill the low 16 bits, odd inputs the high
#     16 bits, two bits each in input order.
#   * Params: entry (nb, g, r) is 4 bytes at ((nb*NG + g)*16 + r)*4: half scale in the
#     low 16 bits, half zero in the high 16 bits.
#   * Padding rows and padding inputs hold code 0 and params (0, 0).
# ----------------------------------------------------------------------------------------
def code_bit(e: int) -> int:
    """Bit position of code e (0..15) inside its 32-bit word."""
    return 16 * (e % 2) + 2 * (e // 2)


def blob_geometry(N: int, K: int, group: int, slices: int) -> dict:
    nb = -(-N // 16)
    kb = -(-K // 256)
    ng = kb * 256 // group
    codes_bytes = nb * kb * 1024
    params_bytes = nb * ng * 64
    a256 = lambda v: -(-v // 256) * 256
    stride = a256(codes_bytes) + a256(params_bytes)
    return {"NB": nb, "KB": kb, "NG": ng, "codes_bytes": codes_bytes,
            "params_bytes": params_bytes, "params_offset": a256(codes_bytes),
            "slice_stride": stride, "total_bytes": stride * slices}


def to_blob(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray, group: int) -> np.ndarray:
    """Write logical codes / params into the packed blob (uint8 array) element by element."""
    S, N, K = codes.shape
    geo = blob_geometry(N, K, group, S)
    KB, NG = geo["KB"], geo["NG"]
    blob = np.zeros(geo["total_bytes"], np.uint8)
    words = blob.view(np.uint32)          # little-endian host, as the device
    halves = blob.view(np.uint16)
    ngr = K // group
    for j in range(S):
        base = j * geo["slice_stride"]
        # codes: loop over (row, 16-input chunk); build each word from its 16 codes
        for n in range(N):
            nb, r = divmod(n, 16)
            for k0 in range(0, K, 16):
                kb, rem = divmod(k0, 256)
                i, c16 = divmod(rem, 64)
                c = c16 // 16
                w = 0
                for e in range(16):
                    w |= int(codes[j, n, k0 + e]) << code_bit(e)
                lane = 16 * c + r
                off = base + (nb * KB + kb) * 1024 + 16 * lane + 4 * i
                words[off // 4] = w
        pbase = base + geo["params_offset"]
        for n in range(N):
            nb, r = divmod(n, 16)
            for g in range(ngr):
                off = pbase + ((nb * NG + g) * 16 + r) * 4
                halves[off // 2] = scale[j, n, g].view(np.uint16)
                halves[off // 2 + 1] = zero[j, n, g].view(np.uint16)
    return blob


def to_blob_fast(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray, group: int) -> np.ndarray:
    """Same bytes as :func:`to_blob`, built with array indexing (for large matrices).

    Equal to ``to_blob`` by test on small shapes; used only where the element loop would
    take minutes.
    """
    S, N, K = codes.shape
    geo = blob_geometry(N, K, group, S)
    NB, KB, NG = geo["NB"], geo["KB"], geo["NG"]
    Np, Kp = NB * 16, KB * 256
    blob = np.zeros(geo["total_bytes"], np.uint8)
    ngr = K // group
    for j in range(S):
        c = np.zeros((Np, Kp), np.uint32)
        c[:N, :K] = codes[j]
        # word value for each (row, 16-chunk)
        c = c.reshape(Np, Kp // 16, 16)
        w = np.zeros((Np, Kp // 16), np.uint32)
        for e in range(16):
            w |= c[:, :, e] << np.uint32(code_bit(e))
        # (nb, r, kb, i, c) -> tile (nb, kb), lane 16c + r, word i
        w = w.reshape(NB, 16, KB, 4, 4)            # nb, r, kb, i, c
        w = w.transpose(0, 2, 4, 1, 3)             # nb, kb, c, r, i
        base = j * geo["slice_stride"]
        blob[base:base + geo["codes_bytes"]] = w.reshape(-1).view(np.uint8)
        p = np.zeros((Np, NG, 2), np.uint16)
        p[:N, :ngr, 0] = scale[j].view(np.uint16)
        p[:N, :ngr, 1] = zero[j].view(np.uint16)
        p = p.reshape(NB, 16, NG, 2).transpose(0, 2, 1, 3)   # nb, g, r, (s, z)
        pb = base + geo["params_offset"]
        blob[pb:pb + geo["params_bytes"]] = p.reshape(-1).view(np.uint8)
    return blob


def from_blob(blob: np.ndarray, N: int, K: int, group: int, slices: int):
    """Read logical codes and params back out of a packed blob (element by element)."""
    geo = blob_geometry(N, K, group, slices)
    KB, NG = geo["KB"], geo["NG"]
    words = np.asarray(blob, np.uint8).view(np.uint32)
    halves = np.asarray(blob, np.uint8).view(np.uint16)
    codes = np.zeros((slices, N, K), np.uint8)
    scale = np.zeros((slices, N, K // group), F16)
    zero = np.zeros((slices, N, K // group), F16)
    for j in range(slices):
        base = j * geo["slice_stride"]
        for n in range(N):
            nb, r = divmod(n, 16)
            for k in range(K):
                kb, rem = divmod(k, 256)
                i, rem2 = divmod(rem, 64)
                c, e = divmod(rem2, 16)
                off = base + (nb * KB + kb) * 1024 + 16 * (16 * c + r) + 4 * i
                codes[j, n, k] = (int(words[off // 4]) >> code_bit(e)) & 3
        pbase = base + geo["params_offset"]
        for n in range(N):
            nb, r = divmod(n, 16)
            for g in range(K // group):
                off = pbase + ((nb * NG + g) * 16 + r) * 4
                scale[j, n, g] = halves[off // 2:off // 2 + 1].view(F16)[0]
                zero[j, n, g] = halves[off // 2 + 1:off // 2 + 2].view(F16)[0]
    return codes, scale, zero
