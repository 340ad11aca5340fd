"""Plain fp64 CPU oracle for N:M and V:N:M pruning, compression and sparse matmul.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The product path (the
HIP library and its Python binding) never imports, links or calls it, and this
module imports nothing from the product package.

Everything here is written to be checked by eye against the pages, not to be
fast: decode the raw bits to float64, apply the selection rule as it is stated,
and compute matrix products by their definition.

Sources (page title, section):
  [ESPLAG]  "Success story: ESPLAG" (inno4scale), Highlights and Research Topic
            (gradual *magnitude* pruning, semi-structured), Solution (N:M
            pruning, the VENOM compressed storage format, the Spatha SpMM
            library; the three figures are missing from the page).
  [SLOPE]   NSF PAR award 2340011 listing, SLOPE abstract (double-pruned
            backward pass: the transposed weight is re-pruned with N:M; lazy
            low-rank adapters added to the sparse weight late in training).
  [2:4+]    "To 2:4 Sparsity and Beyond: Neuron-level Activation Function to
            Accelerate LLM Pre-Training", abstract (2:4 weights and v:n:m
            (Venom) activations in every FFN matmul).
  [SFL]     "Sparser, Faster, Lighter Transformer Language Models",
            Methodologie, training strategy (ReLU instead of SiLU).

Readings taken where the pages are silent:
  * groups are M consecutive elements along the reduction dimension K of the
    left (sparse) operand, starting at k = 0; partial groups are not allowed;
  * the magnitude key is |stored value| in the input dtype; ties go to the
    lower index (positions and V:N:M columns alike); a group keeps exactly N
    survivors even when some are zero;
  * positions are stored with b = ceil(log2 M) bits each, as one LSB-first
    bit stream per row: survivor s of group g sits at bit (g*N + s)*b, and a
    row takes ceil((K/M)*N*b/8) bytes.  For 2:4 that is one nibble per group,
    p0 | p1 << 2, even groups in the low nibble;
  * V:N:M keeps 4 of every M columns per V-row block, ranked by the block's
    column L1 norm (fp64, summed over the V rows in ascending order), then
    2:4 within those 4 columns per row; column choices are stored as u8
    [R/V][K/M][4] ascending, per-row choices as 2:4 nibbles over j = 0..3;
  * ReLU maps every z <= 0 (and -0.0) to +0.0; decompression fills +0.0;
  * the double-pruned transpose re-prunes the already pruned weight W_s;
  * a compress call whose mask keeps a count other than N in a group stores
    +0.0 values at positions 0..N-1 for that group and counts the group.
  * the low-rank adapter is a pair of dense factors U [R, r], Vt [r, K] in the
    weight's dtype; the adapted layer computes W_s @ B + U @ (Vt @ B), with the
    adapter's inner activations Vt @ B formed first and returned as well.
"""

from __future__ import annotations

import math

import numpy as np

F32 = "f32"
BF16 = "bf16"


# ---------------------------------------------------------------------------
# raw bits <-> float64
# ---------------------------------------------------------------------------

def decode(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of every element of a raw array.

    bf16 arrays are uint16 bit patterns: the upper half of an IEEE fp32, so the
    value is the fp32 with those 16 bits on top and zeros below.  fp32 arrays
    are float32.  Both widen to float64 without rounding.
    """
    if dtype == BF16:
        assert raw.dtype == np.uint16
        return (raw.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == F32:
        assert raw.dtype == np.float32
        return raw.astype(np.float64)
    raise ValueError(dtype)


def encode_bf16(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of float64 values, rounded to the nearest bf16 with ties to even.

    bf16 keeps fp32's sign and 8 exponent bits and 8 significant bits (7 stored).  For a finite
    nonzero x = f * 2**e with 0.5 <= |f| < 1 (frexp), the bf16 numbers near x are the multiples of
    2**(e - 8) (of 2**-133 below the normal range, where e - 8 < -133); x is divided by that step,
    rounded half to even (numpy's rounding) and multiplied back, which is exact in float64.  A
    result of 2**128 or more in magnitude is infinity.  Used for products stored in bf16.
    """
    x = np.asarray(x, np.float64)
    _check_finite(x)
    f, e = np.frexp(x)
    step_exp = np.maximum(e - 8, -133)
    y = np.round(np.ldexp(x, -step_exp)) * np.ldexp(1.0, step_exp)     # exact: |quotient| < 2**9
    with np.errstate(over="ignore"):
        y32 = np.where(np.abs(y) >= 2.0 ** 128, np.copysign(np.inf, y), y).astype(np.float32)
    return (y32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def zeros_raw(shape, dtype: str) -> np.ndarray:
    """+0.0 in the raw representation (all bits clear)."""
    return np.zeros(shape, np.uint16 if dtype == BF16 else np.float32)


def _check_finite(x: np.ndarray) -> None:
    if not np.all(np.isfinite(x)):
        raise ValueError("the oracle only accepts finite inputs")


def meta_bits(M: int) -> int:
    """Bits per stored position: ceil(log2 M)."""
    return max(1, math.ceil(math.log2(M)))


def meta_row_bytes(K: int, N: int, M: int) -> int:
    """Bytes of position metadata per row for K columns in N:M groups."""
    return -(-((K // M) * N * meta_bits(M)) // 8)


# ---------------------------------------------------------------------------
# N:M magnitude selection  [ESPLAG Highlights / Solution; 2:4+ abstract]
# ---------------------------------------------------------------------------

def nm_select(keys: np.ndarray, N: int, M: int) -> np.ndarray:
    """Keep N of every M consecutive keys per row: the largest, lower index on ties.

    For positions p = 0..M-1 of one group, rank(p) = #{q : key_q > key_p}
    + #{q < p : key_q == key_p}; p is kept iff rank(p) < N.  Returns a uint8
    mask of the keys' shape.
    """
    R, K = keys.shape
    assert K % M == 0 and 0 < N <= M
    g = keys.reshape(R, K // M, M)
    rank = np.zeros(g.shape, np.int64)
    for p in range(M):
        for q in range(M):
            if q == p:
                continue
            rank[:, :, p] += g[:, :, q] > g[:, :, p]
            if q < p:
                rank[:, :, p] += g[:, :, q] == g[:, :, p]
    return (rank < N).astype(np.uint8).reshape(R, K)


def prune_nm(raw: np.ndarray, dtype: str, N: int, M: int) -> np.ndarray:
    """Magnitude N:M prune of a row-major matrix along its columns -> uint8 mask."""
    x = decode(raw, dtype)
    _check_finite(x)
    return nm_select(np.abs(x), N, M)


# ---------------------------------------------------------------------------
# compressed storage: values + bit-packed positions  [ESPLAG Solution]
# ---------------------------------------------------------------------------

def pack_positions(pos: np.ndarray, M: int, nbytes: int) -> np.ndarray:
    """Positions [R, F] -> uint8 [R, nbytes]: one LSB-first stream of b-bit fields per row.

    Field i occupies bits i*b .. i*b+b-1 of the row, bit j of the stream being
    bit (j % 8) of byte j // 8.
    """
    R, F = pos.shape
    b = meta_bits(M)
    bits = np.zeros((R, nbytes * 8), np.uint8)
    for t in range(b):
        bits[:, t:F * b:b] = (pos >> t) & 1
    return np.packbits(bits, axis=1, bitorder="little")


def unpack_positions_flat(meta: np.ndarray, F: int, M: int) -> np.ndarray:
    """Inverse of pack_positions: uint8 [R, nbytes] -> positions [R, F]."""
    b = meta_bits(M)
    bits = np.unpackbits(meta, axis=1, bitorder="little").astype(np.int64)
    pos = np.zeros((meta.shape[0], F), np.int64)
    for t in range(b):
        pos += bits[:, t:F * b:b] << t
    return pos


def compress_nm(raw: np.ndarray, mask: np.ndarray, N: int, M: int):
    """Gather each group's kept elements in ascending position and pack positions.

    Returns (values, meta, bad_groups): values [R, K/M*N] hold the raw bits of
    the kept elements, meta [R, meta_row_bytes] the packed positions.  A group
    whose mask keeps a count other than N is stored as +0.0 values at
    positions 0..N-1 and counted in bad_groups.
    """
    R, K = raw.shape
    G = K // M
    mg = (mask.reshape(R, G, M) != 0)
    count = mg.sum(axis=2)
    bad = count != N
    # kept positions in ascending order: a stable sort puts kept (0) before dropped (1)
    pos = np.argsort((~mg).astype(np.int8), axis=2, kind="stable")[:, :, :N]
    pos[bad] = np.arange(N)
    vals = np.take_along_axis(raw.reshape(R, G, M), pos, axis=2)
    vals[bad] = 0
    meta = pack_positions(pos.reshape(R, G * N), M, meta_row_bytes(K, N, M))
    return vals.reshape(R, G * N), meta, int(bad.sum())


def unpack_positions(meta: np.ndarray, R: int, K: int, N: int, M: int) -> np.ndarray:
    """Positions [R, K/M, N] from the packed metadata."""
    G = K // M
    return unpack_positions_flat(meta, G * N, M).reshape(R, G, N)


def decompress_nm(values: np.ndarray, meta: np.ndarray, R: int, K: int, N: int, M: int) -> np.ndarray:
    """Dense raw matrix: +0.0 everywhere, kept values placed at their positions."""
    G = K // M
    pos = unpack_positions(meta, R, K, N, M)
    out = np.zeros((R, G, M), values.dtype)
    np.put_along_axis(out, pos, values.reshape(R, G, N), axis=2)
    return out.reshape(R, K)


# ---------------------------------------------------------------------------
# V:N:M (VENOM) activation/weight pruning  [2:4+ abstract; ESPLAG Solution;
# SFL Methodologie for ReLU]
# ---------------------------------------------------------------------------

VNM_KEEP_COLS = 4  # columns kept per M-group in a V-row block (then 2:4 inside)


def relu_raw(raw: np.ndarray, dtype: str) -> np.ndarray:
    """ReLU on raw bits: values > 0 keep their bits, everything else becomes +0.0."""
    x = decode(raw, dtype)
    out = raw.copy()
    out[~(x > 0)] = 0
    return out


def venom_column_l1(x: np.ndarray, V: int, M: int) -> np.ndarray:
    """Column L1 norms per V-row block: [R/V, K] in fp64, rows added in ascending order."""
    R, K = x.shape
    out = np.zeros((R // V, K), np.float64)
    for blk in range(R // V):
        acc = np.zeros(K, np.float64)
        for r in range(blk * V, (blk + 1) * V):
            acc = acc + np.abs(x[r])
        out[blk] = acc
    return out


def prune_venom(raw: np.ndarray, dtype: str, V: int, M: int, apply_relu: bool):
    """V:N:M prune (N = 2) and compress.

    Per V-row block and M-column group: keep the 4 columns with the largest
    block L1 norm (lower column on ties); then, per row, keep 2 of those 4 by
    magnitude (lower j on ties).  Returns (values [R, K/M*2], meta
    [R, K/(2M)] nibbles j0 | j1 << 2, colsel u8 [R/V, K/M, 4], mask [R, K],
    h) where h is the (ReLU'd) raw input the selection ran on.
    """
    R, K = raw.shape
    assert R % V == 0 and K % M == 0 and M >= VNM_KEEP_COLS
    h = relu_raw(raw, dtype) if apply_relu else raw.copy()
    x = decode(h, dtype)
    _check_finite(x)
    G = K // M
    l1 = venom_column_l1(x, V, M)                                   # [R/V, K]
    colmask = nm_select(l1, VNM_KEEP_COLS, M)                       # [R/V, K]
    colsel = np.zeros((R // V, G, VNM_KEEP_COLS), np.uint8)
    for blk in range(R // V):
        for g in range(G):
            colsel[blk, g] = np.nonzero(colmask[blk, g * M:(g + 1) * M])[0]
    # gather the 4 selected columns of every group for every row
    cols = (np.arange(G)[:, None] * M + colsel.astype(np.int64))    # [R/V, G, 4]
    cols_rows = np.repeat(cols, V, axis=0).reshape(R, G * VNM_KEEP_COLS)
    sub_raw = np.take_along_axis(h, cols_rows, axis=1)              # [R, G*4]
    sub_mask = nm_select(np.abs(decode(sub_raw, dtype)), 2, VNM_KEEP_COLS)
    values, meta, bad = compress_nm(sub_raw, sub_mask, 2, VNM_KEEP_COLS)
    assert bad == 0
    mask = np.zeros((R, K), np.uint8)
    rows = np.arange(R)[:, None]
    mask[np.broadcast_to(rows, cols_rows.shape), cols_rows] = sub_mask
    return values, meta, colsel, mask, h


def decompress_venom(values: np.ndarray, meta: np.ndarray, colsel: np.ndarray,
                     R: int, K: int, V: int, M: int) -> np.ndarray:
    """Dense raw [R, K] from V:N:M values, nibbles and column selections."""
    G = K // M
    sub = decompress_nm(values, meta, R, G * VNM_KEEP_COLS, 2, VNM_KEEP_COLS)  # [R, G*4]
    cols = np.repeat(colsel.astype(np.int64), V, axis=0)                       # [R, G, 4]
    out = np.zeros((R, G, M), values.dtype)
    np.put_along_axis(out, cols, sub.reshape(R, G, VNM_KEEP_COLS), axis=2)
    return out.reshape(R, K)


# ---------------------------------------------------------------------------
# double pruning of the transposed weight  [SLOPE abstract]
# ---------------------------------------------------------------------------

def reprune_t(values: np.ndarray, meta: np.ndarray, R: int, K: int, dtype: str):
    """W_s (2:4 along K, compressed) -> W_ds^T (2:4 along the former rows R).

    W_s is decompressed with +0.0 fill, transposed to [K, R], pruned 2:4 by
    magnitude along R and compressed.  Returns (values_t [K, R/2],
    meta_t [K, R/8]).
    """
    ws = decompress_nm(values, meta, R, K, 2, 4)
    wt = np.ascontiguousarray(ws.T)
    mask_t = prune_nm(wt, dtype, 2, 4)
    vt, mt, bad = compress_nm(wt, mask_t, 2, 4)
    assert bad == 0
    return vt, mt


# ---------------------------------------------------------------------------
# sparse x dense products: the plain definitions  [ESPLAG Research Topic
# (SpMM); 2:4+ abstract (all FFN matmuls); SLOPE abstract (backward)]
# ---------------------------------------------------------------------------

def spmm_nm(values, meta, R, K, B_raw, dtype):
    """C = decompress(values, meta) @ B in float64 (2:4)."""
    A = decode(decompress_nm(values, meta, R, K, 2, 4), dtype)
    B = decode(B_raw, dtype)
    return A @ B


def spmm_nm_loop(values, meta, R, K, B_raw, dtype):
    """Same product as spmm_nm, by the explicit gather loop (small inputs only).

    C[r, n] = sum over groups g and slots s of values[r, 2g+s] * B[4g + p_s, n].
    """
    pos = unpack_positions(meta, R, K, 2, 4)
    v = decode(values, dtype)
    B = decode(B_raw, dtype)
    Nc = B.shape[1]
    C = np.zeros((R, Nc))
    for r in range(R):
        for n in range(Nc):
            acc = 0.0
            for g in range(K // 4):
                for s in range(2):
                    acc += v[r, 2 * g + s] * B[4 * g + pos[r, g, s], n]
            C[r, n] = acc
    return C


def spmm_nm_general(values, meta, R, K, N, M, B_raw, dtype):
    """C = decompress(values, meta) @ B in float64 for any N:M compressed matrix."""
    A = decode(decompress_nm(values, meta, R, K, N, M), dtype)
    return A @ decode(B_raw, dtype)


def spmm_nm_general_loop(values, meta, R, K, N, M, B_raw, dtype):
    """Same product by the explicit gather loop (small inputs only).

    C[r, n] = sum over groups g and slots s of values[r, N*g+s] * B[M*g + p_s, n].
    """
    pos = unpack_positions(meta, R, K, N, M)
    v = decode(values, dtype)
    B = decode(B_raw, dtype)
    C = np.zeros((R, B.shape[1]))
    for r in range(R):
        for n in range(B.shape[1]):
            acc = 0.0
            for g in range(K // M):
                for s in range(N):
                    acc += v[r, N * g + s] * B[M * g + pos[r, g, s], n]
            C[r, n] = acc
    return C


def spmm_venom(values, meta, colsel, R, K, V, M, B_raw, dtype):
    """C = decompress_venom(...) @ B in float64."""
    A = decode(decompress_venom(values, meta, colsel, R, K, V, M), dtype)
    return A @ decode(B_raw, dtype)


def spmm_venom_loop(values, meta, colsel, R, K, V, M, B_raw, dtype):
    """C[r, n] = sum_g sum_s values[r, 2g+s] * B[g*M + colsel[r//V, g, j_s], n] (small inputs)."""
    G = K // M
    pos = unpack_positions(meta, R, G * VNM_KEEP_COLS, 2, VNM_KEEP_COLS)
    v = decode(values, dtype)
    B = decode(B_raw, dtype)
    C = np.zeros((R, B.shape[1]))
    for r in range(R):
        for n in range(B.shape[1]):
            acc = 0.0
            for g in range(G):
                for s in range(2):
                    col = g * M + int(colsel[r // V, g, pos[r, g, s]])
                    acc += v[r, 2 * g + s] * B[col, n]
            C[r, n] = acc
    return C


def sddmm_nm(D_raw, X_raw, meta, R, Kc, dtype):
    """dW values [R, Kc/2]: (D @ X^T) in float64 read at the kept positions of meta (2:4)."""
    full = decode(D_raw, dtype) @ decode(X_raw, dtype).T           # [R, Kc]
    pos = unpack_positions(meta, R, Kc, 2, 4)
    cols = (np.arange(Kc // 4)[None, :, None] * 4 + pos).reshape(R, Kc // 2)
    return np.take_along_axis(full, cols, axis=1)


def sddmm_nm_rows(D_raw, X_raw, meta, rows, Kc, dtype):
    """sddmm_nm restricted to the given rows of D (for sampled checks at full size)."""
    D = decode(D_raw[rows], dtype)
    full = D @ decode(X_raw, dtype).T
    pos = unpack_positions(meta[rows], len(rows), Kc, 2, 4)
    cols = (np.arange(Kc // 4)[None, :, None] * 4 + pos).reshape(len(rows), Kc // 2)
    return np.take_along_axis(full, cols, axis=1)


# ---------------------------------------------------------------------------
# backward of the V:N:M down-projection  [2:4+ abstract: v:n:m activations in
# every FFN matmul; SFL Methodologie: ReLU activations]
#
# Forward: Y = h_s @ W_down, h_s = the V:N:M form of h = ReLU(z) [T, F] (V-row
# blocks of tokens, groups of M along F).  Readings (the pages give only the
# forward idea): the gradient reaches z only through the entries the forward
# kept, times ReLU's derivative (1 where the kept activation is > 0, 0 where it
# is +0.0, i.e. z <= 0); the weight gradient is dW_down = h_s^T @ dY.
# ---------------------------------------------------------------------------

def venom_kept_columns(meta, colsel, T, F, V, M):
    """Dense column index [T, (F/M)*2] of every kept entry: g*M + colsel[t//V, g, j_s]."""
    G = F // M
    pos = unpack_positions(meta, T, G * VNM_KEEP_COLS, 2, VNM_KEEP_COLS)          # [T, G, 2] = j_s
    sel = np.repeat(colsel.astype(np.int64), V, axis=0)                           # [T, G, 4]
    cols = np.arange(G)[None, :, None] * M + np.take_along_axis(sel, pos, axis=2)  # [T, G, 2]
    return cols.reshape(T, G * 2)


def sddmm_venom(dY_raw, Wd_raw, h_values, h_meta, h_colsel, T, F, V, M, dtype, relu):
    """dZ values [T, (F/M)*2], aligned with h_s's values: (dY @ W_down^T) in float64 read at
    h_s's kept positions, times ReLU's derivative at them when relu."""
    full = decode(dY_raw, dtype) @ decode(Wd_raw, dtype).T                        # [T, F]
    out = np.take_along_axis(full, venom_kept_columns(h_meta, h_colsel, T, F, V, M), axis=1)
    if relu:
        out = np.where(decode(h_values, dtype) > 0, out, 0.0)
    return out


def sddmm_venom_loop(dY_raw, Wd_raw, h_values, h_meta, h_colsel, T, F, V, M, dtype, relu):
    """sddmm_venom element by element (small inputs)."""
    G = F // M
    pos = unpack_positions(h_meta, T, G * VNM_KEEP_COLS, 2, VNM_KEEP_COLS)
    dY, Wd, hv = decode(dY_raw, dtype), decode(Wd_raw, dtype), decode(h_values, dtype)
    out = np.zeros((T, 2 * G))
    for t in range(T):
        for g in range(G):
            for s in range(2):
                col = g * M + int(h_colsel[t // V, g, pos[t, g, s]])
                acc = 0.0
                for c in range(dY.shape[1]):
                    acc += dY[t, c] * Wd[col, c]
                out[t, 2 * g + s] = acc if (not relu or hv[t, 2 * g + s] > 0) else 0.0
    return out


def spmm_venom_tn(h_values, h_meta, h_colsel, T, F, V, M, dY_raw, dtype):
    """dW_down [F, Nc] = decompress_venom(h_s)^T @ dY in float64."""
    H = decode(decompress_venom(h_values, h_meta, h_colsel, T, F, V, M), dtype)
    return H.T @ decode(dY_raw, dtype)


def spmm_venom_tn_loop(h_values, h_meta, h_colsel, T, F, V, M, dY_raw, dtype):
    """dW_down[col] += h_s[t, 2g+s] * dY[t] for every kept entry (small inputs)."""
    G = F // M
    pos = unpack_positions(h_meta, T, G * VNM_KEEP_COLS, 2, VNM_KEEP_COLS)
    hv, dY = decode(h_values, dtype), decode(dY_raw, dtype)
    out = np.zeros((F, dY.shape[1]))
    for t in range(T):
        for g in range(G):
            for s in range(2):
                col = g * M + int(h_colsel[t // V, g, pos[t, g, s]])
                out[col] += hv[t, 2 * g + s] * dY[t]
    return out


# ---------------------------------------------------------------------------
# gradual magnitude pruning schedule  [ESPLAG Highlights, Research Topic
# (semi-structured gradual magnitude pruning); 2:4+ abstract (sparse steps,
# then regular dense steps towards the end)]
#
# Reading (the pages give no schedule): dense before the ramp; pruning events
# every `interval` steps from t_begin through t_end; the kept count per group
# falls linearly (the removed count rounded up) from M
# to n_final over the events; the last pattern holds until the dense switch at
# t_dense (none when t_dense < 0).
# ---------------------------------------------------------------------------

def gmp_n_at(M, n_final, t_begin, t_end, interval, t_dense, step):
    """(N in effect at `step` -- M when dense --, whether `step` is a pruning event)."""
    if step < t_begin or (t_dense >= 0 and step >= t_dense):
        return M, False
    event_steps = list(range(t_begin, t_end + 1, interval))
    E = len(event_steps)
    done = [s for s in event_steps if s <= step]                  # events so far, this one included
    e = len(done) - 1
    removed = -((-(M - n_final) * (e + 1)) // E)                  # ceil((M - n_final)(e + 1) / E)
    return M - removed, step in event_steps


# ---------------------------------------------------------------------------
# sparse plus low-rank  [SLOPE abstract: low-rank adapters joined to the sparse
# weight for the last iterations of pre-training, at little extra cost]
# ---------------------------------------------------------------------------

def spmm_nm_lowrank(values, meta, R, K, B_raw, U_raw, Vt_raw, dtype):
    """Sparse weight plus a low-rank adapter, applied lazily, in float64.

    The adapted weight is W_s + U @ Vt (U [R, r], Vt [r, K]); it is never formed.
    The adapter's inner activations T = Vt @ B [r, Nc] are computed first, then
    C = decompress(values, meta) @ B + U @ T.  Returns (C, T).
    """
    T = decode(Vt_raw, dtype) @ decode(B_raw, dtype)
    C = spmm_nm(values, meta, R, K, B_raw, dtype) + decode(U_raw, dtype) @ T
    return C, T


def spmm_nm_lowrank_rows(values, meta, rows, K, B_raw, U_raw, Vt_raw, dtype):
    """spmm_nm_lowrank restricted to the given rows of the output (sampled checks at full size)."""
    A = decode(decompress_nm(values[rows], meta[rows], len(rows), K, 2, 4), dtype)
    B = decode(B_raw, dtype)
    T = decode(Vt_raw, dtype) @ B
    return A @ B + decode(U_raw[rows], dtype) @ T


# ---------------------------------------------------------------------------
# the acceptance test for floating-point results
# ---------------------------------------------------------------------------

def abs_bound(A64: np.ndarray, B64: np.ndarray) -> np.ndarray:
    """(|A| @ |B|) in float64: the per-element scale of the rounding error bound."""
    return np.abs(A64) @ np.abs(B64)


def within_tolerance(C: np.ndarray, C_ref: np.ndarray, bound: np.ndarray,
                     rel_fro: float = 1e-3, elem: float = 1e-2):
    """Relative Frobenius error <= rel_fro and |C - C_ref| <= elem * bound elementwise."""
    C = np.asarray(C, np.float64)
    err = np.abs(C - C_ref)
    ref_norm = np.linalg.norm(C_ref)
    fro = np.linalg.norm(C - C_ref) / ref_norm if ref_norm > 0 else np.linalg.norm(C - C_ref)
    elem_ok = bool(np.all(err <= elem * bound))
    return bool(fro <= rel_fro and elem_ok), float(fro), float(np.max(err - elem * bound, initial=-np.inf))
