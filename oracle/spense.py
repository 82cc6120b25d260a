"""Plain NumPy oracle of the Spense linear layer (test infrastructure only).

Notation: W[N,K] weights, X[M,K] activations, D the dense column set with
K_d = |D| columns, K_s = K - K_d sparse columns, pi the column order
[sparse columns ascending | dense columns ascending], X' = X[:, pi].

Sources (all on the SpenseGPT gist.science explainer unless noted):
  * Technical Summary 2.A "The Spense Format": one contiguous dense region
    plus one contiguous 2:4 region; input-split accumulates the sparse-GEMM and
    dense-GEMM results into the same output.
  * Technical Summary 2.B: SpenseGPT keeps the last p% of indices dense;
    SpenseGPT+ chooses an index set and moves it into the contiguous dense
    block by a permutation, which leaves the product unchanged.
  * Technical Summary 1 (and SlideSparse explainer, Technical summary 1):
    a 2:4 group of four consecutive weights holds at most two nonzeros.
Readings where the pages are silent (tie-break, metadata encoding, fp8
magnitude domain, fraction rounding) are the ones listed in the design notes:
magnitude = stored bit pattern with the sign cleared, equal magnitudes go to
the lower in-group position, the nibble for a group is i0 | i1 << 2 with
i0 < i1, eight groups per uint32 word starting at the low nibble, and
K_d = round-half-away(p * K).
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

DT_F32 = 0
DT_BF16 = 1
DT_FP8 = 2


class DenseSetError(ValueError):
    """Raised for a dense set or fraction the format cannot represent."""


# ---------------------------------------------------------------------------
# a1: dense-set resolution  (Technical Summary 2.A / 2.B)
# ---------------------------------------------------------------------------
def resolve_dense_set(K: int, dense_cols=None, dense_fraction: Optional[float] = None):
    """Return (pi, K_s, K_d).

    With ``dense_cols`` the given set is the dense region (SpenseGPT+ style:
    arbitrary indices, moved into one contiguous block).  Otherwise the dense
    region is the last K_d = round(p*K) indices (SpenseGPT: the last p%).
    pi lists the sparse indices ascending, then the dense indices ascending.
    The sparse region must hold whole groups of four.
    """
    if K <= 0:
        raise DenseSetError("K must be positive")
    if dense_cols is not None:
        D = np.asarray(dense_cols, dtype=np.int64).ravel()
        if D.size and (D.min() < 0 or D.max() >= K):
            raise DenseSetError("dense column out of range")
        if np.unique(D).size != D.size:
            raise DenseSetError("duplicate dense column")
        D = np.sort(D)
    else:
        if dense_fraction is None:
            raise DenseSetError("need dense_cols or dense_fraction")
        p = float(dense_fraction)
        if not (0.0 <= p <= 1.0):
            raise DenseSetError("dense_fraction outside [0, 1]")
        K_d = int(math.floor(p * K + 0.5))
        D = np.arange(K - K_d, K, dtype=np.int64)
    K_d = int(D.size)
    K_s = K - K_d
    if K_s % 4 != 0:
        raise DenseSetError("sparse region length must be a multiple of 4")
    is_dense = np.zeros(K, dtype=bool)
    is_dense[D] = True
    sparse = np.nonzero(~is_dense)[0]
    pi = np.concatenate([sparse, D]).astype(np.int64)
    return pi, K_s, K_d


# ---------------------------------------------------------------------------
# element encodings
# ---------------------------------------------------------------------------
def magnitude_key(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Magnitude order key: the stored bit pattern with its sign bit cleared.

    For IEEE-style encodings (fp32, bf16, e4m3fn) this unsigned integer orders
    finite magnitudes exactly as their values do; +0 and -0 compare equal.
    """
    if dtype == DT_F32:
        u = np.ascontiguousarray(bits, dtype=np.float32).view(np.uint32)
        return (u & np.uint32(0x7FFFFFFF)).astype(np.int64)
    if dtype == DT_BF16:
        return (np.asarray(bits, dtype=np.uint16) & np.uint16(0x7FFF)).astype(np.int64)
    if dtype == DT_FP8:
        return (np.asarray(bits, dtype=np.uint8) & np.uint8(0x7F)).astype(np.int64)
    raise ValueError(f"unknown dtype {dtype}")


def _e4m3_value(code: int) -> float:
    """OCP e4m3fn: sign, 4-bit exponent (bias 7), 3-bit mantissa; S.1111.111 is NaN."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode_values(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Stored bits -> float64 values."""
    if dtype == DT_F32:
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    if dtype == DT_BF16:
        u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
        with np.errstate(invalid="ignore"):
            return u.view(np.float32).astype(np.float64)
    if dtype == DT_FP8:
        return _E4M3_TABLE[np.asarray(bits, dtype=np.uint8)]
    raise ValueError(f"unknown dtype {dtype}")


def _storage_dtype(dtype: int):
    return {DT_F32: np.float32, DT_BF16: np.uint16, DT_FP8: np.uint8}[dtype]


# ---------------------------------------------------------------------------
# a2 + a3: 2:4 magnitude selection and compression, dense block copy
# ---------------------------------------------------------------------------
@dataclass
class Packed:
    """Canonical packed form of one weight matrix.

    vals  [N, K_s/2]          kept values (bit copies), two per group, lower position first
    meta  [N, ceil(K_s/32)]   uint32; group g's nibble (i0 | i1<<2) at bits 4*(g%8) of word g//8
    mask  [N, K_s]            uint8 0/1, 1 on kept slots (columns in pi order)
    dense [N, K_d]            bit copies of W[:, pi[K_s:]]
    pi    [K]                 column order
    """

    vals: np.ndarray
    meta: np.ndarray
    mask: np.ndarray
    dense: np.ndarray
    pi: np.ndarray
    K_s: int
    K_d: int
    dtype: int


def pack(W: np.ndarray, dtype: int, pi: np.ndarray, K_s: int) -> Packed:
    """Choose the 2:4 mask by magnitude and compress the sparse region.

    Group g of row n holds the four sparse-region columns pi[4g..4g+3].  The two
    slots with the largest magnitude key are kept; among equal keys the lower
    slot wins (a stable sort of the negated keys realises exactly this order).
    """
    W = np.asarray(W)
    N, K = W.shape
    if K_s % 4 != 0:
        raise DenseSetError("sparse region length must be a multiple of 4")
    G = K_s // 4
    pi = np.asarray(pi, dtype=np.int64)
    Ws = W[:, pi[:K_s]].reshape(N, G, 4)
    keys = magnitude_key(Ws, dtype)
    order = np.argsort(-keys, axis=2, kind="stable")[:, :, :2]
    i0 = order.min(axis=2)
    i1 = order.max(axis=2)
    mask = np.zeros((N, G, 4), dtype=np.uint8)
    np.put_along_axis(mask, i0[:, :, None], 1, axis=2)
    np.put_along_axis(mask, i1[:, :, None], 1, axis=2)
    v0 = np.take_along_axis(Ws, i0[:, :, None], axis=2)[:, :, 0]
    v1 = np.take_along_axis(Ws, i1[:, :, None], axis=2)[:, :, 0]
    vals = np.empty((N, 2 * G), dtype=W.dtype)
    vals[:, 0::2] = v0
    vals[:, 1::2] = v1
    nib = (i0 | (i1 << 2)).astype(np.uint64)
    n_words = (G + 7) // 8
    meta = np.zeros((N, n_words), dtype=np.uint64)
    for j in range(8):
        part = nib[:, j::8]
        meta[:, : part.shape[1]] |= part << np.uint64(4 * j)
    dense = np.ascontiguousarray(W[:, pi[K_s:]])
    return Packed(vals=vals, meta=meta.astype(np.uint32), mask=mask.reshape(N, K_s),
                  dense=dense, pi=pi, K_s=K_s, K_d=K - K_s, dtype=dtype)


def unpack_bits(p: Packed) -> np.ndarray:
    """Rebuild W with pruned positions set to (+0) from vals/meta/dense, natural column order."""
    N = p.vals.shape[0]
    K = p.pi.size
    G = p.K_s // 4
    out = np.zeros((N, K), dtype=_storage_dtype(p.dtype))
    if G:
        g = np.arange(G)
        nib = (p.meta[:, g // 8].astype(np.uint64) >> (4 * (g % 8)).astype(np.uint64)) & np.uint64(0xF)
        i0 = (nib & np.uint64(3)).astype(np.int64)
        i1 = (nib >> np.uint64(2)).astype(np.int64)
        rows = np.arange(N)[:, None]
        col0 = p.pi[4 * g[None, :] + i0]
        col1 = p.pi[4 * g[None, :] + i1]
        out[rows, col0] = p.vals[:, 0::2]
        out[rows, col1] = p.vals[:, 1::2]
    if p.K_d:
        out[:, p.pi[p.K_s:]] = p.dense
    return out


def decompress(p: Packed, scales=None) -> np.ndarray:
    """Values of the pruned weight matrix in natural column order, float64 (scale not applied)."""
    return decode_values(unpack_bits(p), p.dtype)


# ---------------------------------------------------------------------------
# a4..a7: the layer output  Y = s * (X' . W_sparse^T + X' . W_dense^T)
# ---------------------------------------------------------------------------
def linear_ref(X_bits: np.ndarray, xdtype: int, p: Packed, scales=None):
    """Exact layer output in float64 and its error scale.

    Since X'[:, j] = X[:, pi[j]] and the packed weights decompress to the same
    columns pi[j], the sparse product plus the dense product equals X times the
    decompressed (pruned) weight matrix in natural order:
        Y[m, n] = s[n] * sum_k X[m, k] * Wp[n, k]
        B[m, n] = s[n] * sum_k |X[m, k] * Wp[n, k]|
    with s = 1 for non-fp8 weights.  Returns (Y, B), both [M, N] float64.
    """
    Wp = decompress(p)
    X = decode_values(X_bits, xdtype)
    Y = X @ Wp.T
    B = np.abs(X) @ np.abs(Wp).T
    if scales is not None:
        s = np.asarray(scales, dtype=np.float32).astype(np.float64)
        Y = Y * s[None, :]
        B = B * s[None, :]
    return Y, B


def dense_linear_ref(X_bits: np.ndarray, xdtype: int, W_bits: np.ndarray, wdtype: int, scales=None):
    """All-dense comparator Y = X . (s o W)^T of the unpruned weights, with its error scale."""
    W = decode_values(W_bits, wdtype)
    X = decode_values(X_bits, xdtype)
    Y = X @ W.T
    B = np.abs(X) @ np.abs(W).T
    if scales is not None:
        s = np.asarray(scales, dtype=np.float32).astype(np.float64)
        Y = Y * s[None, :]
        B = B * s[None, :]
    return Y, B


# ---------------------------------------------------------------------------
# Output-split form (Technical Summary 2.A "The Spense Format": the output is
# split, one part from the sparse GEMM and the other from the dense GEMM; the
# page uses it for the GLU gate and up projections).  The split runs over the
# output rows: a set of dense rows keeps all its weights, every other row is
# 2:4 along K in groups of four consecutive columns.  The two parts write
# different outputs, so nothing is accumulated across them.  As for columns,
# a chosen row set is moved into one contiguous block (Technical Summary 2.B:
# permuting intermediate indices leaves the block's output unchanged, up to
# the same permutation of the output columns).
# ---------------------------------------------------------------------------
def resolve_dense_rows(N: int, K: int, dense_rows=None, dense_fraction: Optional[float] = None):
    """Return (rho, N_s, N_d): rho lists the sparse rows ascending, then the dense rows ascending.

    A fraction p selects the last N_d = round-half-away(p*N) rows (the reading
    used for dense columns).  Sparse rows need K to hold whole groups of four.
    """
    if N <= 0 or K <= 0:
        raise DenseSetError("N and K must be positive")
    if dense_rows is not None:
        D = np.asarray(dense_rows, dtype=np.int64).ravel()
        if D.size and (D.min() < 0 or D.max() >= N):
            raise DenseSetError("dense row out of range")
        if np.unique(D).size != D.size:
            raise DenseSetError("duplicate dense row")
        D = np.sort(D)
    else:
        if dense_fraction is None:
            raise DenseSetError("need dense_rows or dense_fraction")
        p = float(dense_fraction)
        if not (0.0 <= p <= 1.0):
            raise DenseSetError("dense_fraction outside [0, 1]")
        N_d = int(math.floor(p * N + 0.5))
        D = np.arange(N - N_d, N, dtype=np.int64)
    N_d = int(D.size)
    N_s = N - N_d
    if N_s > 0 and K % 4 != 0:
        raise DenseSetError("K must be a multiple of 4 when any row is sparse")
    is_dense = np.zeros(N, dtype=bool)
    is_dense[D] = True
    rho = np.concatenate([np.nonzero(~is_dense)[0], D]).astype(np.int64)
    return rho, N_s, N_d


@dataclass
class PackedRows:
    """Canonical output-split form.

    sparse  Packed of the sparse rows rho[:N_s] (all K columns 2:4, natural column order)
    dense   [N_d, K] bit copies of W[rho[N_s:], :]
    rho     [N] row order
    """

    sparse: Packed
    dense: np.ndarray
    rho: np.ndarray
    N_s: int
    N_d: int
    dtype: int


def pack_rows(W: np.ndarray, dtype: int, rho: np.ndarray, N_s: int) -> PackedRows:
    """2:4 selection on the sparse rows (groups of four consecutive columns), dense rows copied."""
    W = np.asarray(W)
    N, K = W.shape
    rho = np.asarray(rho, dtype=np.int64)
    Ks = K if N_s > 0 else 0
    sp = pack(W[rho[:N_s]], dtype, np.arange(K, dtype=np.int64), Ks)
    dense = np.ascontiguousarray(W[rho[N_s:]])
    return PackedRows(sparse=sp, dense=dense, rho=rho, N_s=N_s, N_d=N - N_s, dtype=dtype)


def unpack_rows_bits(p: PackedRows) -> np.ndarray:
    """Rebuild W with pruned positions (+0) in the natural row and column order."""
    N = p.rho.size
    K = p.dense.shape[1] if p.N_d else p.sparse.pi.size
    out = np.zeros((N, K), dtype=_storage_dtype(p.dtype))
    if p.N_s:
        out[p.rho[: p.N_s]] = unpack_bits(p.sparse)
    if p.N_d:
        out[p.rho[p.N_s:]] = p.dense
    return out


def linear_rows_ref(X_bits: np.ndarray, xdtype: int, p: PackedRows, scales=None):
    """Exact output-split layer output in float64 and its error scale (same definition as linear_ref)."""
    Wp = decode_values(unpack_rows_bits(p), p.dtype)
    X = decode_values(X_bits, xdtype)
    Y = X @ Wp.T
    B = np.abs(X) @ np.abs(Wp).T
    if scales is not None:
        s = np.asarray(scales, dtype=np.float32).astype(np.float64)
        Y = Y * s[None, :]
        B = B * s[None, :]
    return Y, B


# ---------------------------------------------------------------------------
# GLU MLP block (Technical Summary 2.A: output-split for the gate and up
# projections, input-split for the down projection; Technical Summary 2.B:
# the dense intermediate indices can be permuted into one contiguous block
# without changing the block's output).  The gate nonlinearity is SiLU, as in
# the GLU models the page evaluates; the page does not name it.
# ---------------------------------------------------------------------------
def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x) in float64."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):  # exp(-x) = inf for x << 0 gives the limit -0
        return x / (1.0 + np.exp(-x))


def glu_block_ref(X_bits: np.ndarray, xdtype: int, Wg_bits, Wu_bits, Wd_bits, dtype: int, dense_idx,
                  s_g=None, s_u=None, s_d=None):
    """Exact block output in float64.

    D = dense_idx, a set of intermediate indices: rows D of W_gate and W_up
    stay dense (output-split), columns D of W_down stay dense (input-split);
    every other gate/up row is 2:4 along the hidden dimension and every other
    down column group is 2:4 along the intermediate dimension in the order
    [non-dense ascending | dense ascending].
        G = X W_gate'^T (s_g), U = X W_up'^T (s_u), A = silu(G) * U,
        Y = A W_down'^T (s_d)
    Returns dict(G, U, A, Y, B_G, B_U, B_Y) with B_* = the |x||w| error scales
    (B_Y taken over A).
    """
    I = Wg_bits.shape[0]
    rho, I_s, _ = resolve_dense_rows(I, Wg_bits.shape[1], dense_rows=dense_idx)
    G, B_G = linear_rows_ref(X_bits, xdtype, pack_rows(Wg_bits, dtype, rho, I_s), s_g)
    U, B_U = linear_rows_ref(X_bits, xdtype, pack_rows(Wu_bits, dtype, rho, I_s), s_u)
    A = silu(G) * U
    pi, K_s, _ = resolve_dense_set(I, dense_cols=dense_idx)
    Y, B_Y = down_ref(A, pack(Wd_bits, dtype, pi, K_s), s_d)
    return dict(G=G, U=U, A=A, Y=Y, B_G=B_G, B_U=B_U, B_Y=B_Y, rho=rho, I_s=I_s)


def down_ref(A: np.ndarray, p: Packed, scales=None):
    """The down projection on float64 intermediate values A [M, I] (natural index order)."""
    Wp = decompress(p)
    A = np.asarray(A, dtype=np.float64)
    Y = A @ Wp.T
    B = np.abs(A) @ np.abs(Wp).T
    if scales is not None:
        s = np.asarray(scales, dtype=np.float32).astype(np.float64)
        Y = Y * s[None, :]
        B = B * s[None, :]
    return Y, B


# ---------------------------------------------------------------------------
# SpenseGPT+ dense index selection (Technical Summary 2.B): an importance score
# per intermediate index of a GLU block, aggregated over the gate, up and down
# projections; each weight scores S_ij = |W_ij| * sqrt(H_jj) (the magnitude of
# the weight times that of its input), H = X^T X over calibration inputs of
# that projection.  The top-scoring indices stay dense.  Readings: the
# aggregation is a plain sum over the weights attached to index i (row i of
# gate and up, column i of down); |W| is the dequantised magnitude (per-row
# scale included); ties in the top-k go to the lower index.
# ---------------------------------------------------------------------------
def hessian_diag(X_bits: np.ndarray, xdtype: int) -> np.ndarray:
    """diag(X^T X): the sum over calibration rows of each input column squared (float64)."""
    X = decode_values(X_bits, xdtype)
    return np.sum(X * X, axis=0)


def glu_scores_ref(X_cal_bits, A_cal_bits, xdtype: int, Wg_bits, Wu_bits, Wd_bits, dtype: int,
                   s_g=None, s_u=None, s_d=None) -> np.ndarray:
    """score[i] = sum_j |Wg[i,j]| sqrt(Hx_jj) + sum_j |Wu[i,j]| sqrt(Hx_jj) + sum_n |Wd[n,i]| sqrt(Ha_ii).

    X_cal [T, H]: calibration inputs of gate/up; A_cal [T, I]: calibration
    inputs of down (the intermediate activations).  Returns float64 [I].
    """
    def mag(Wb, s):
        Wv = np.abs(decode_values(Wb, dtype))
        if s is not None:
            Wv = Wv * np.abs(np.asarray(s, dtype=np.float32).astype(np.float64))[:, None]
        return Wv
    rx = np.sqrt(hessian_diag(X_cal_bits, xdtype))
    ra = np.sqrt(hessian_diag(A_cal_bits, xdtype))
    return mag(Wg_bits, s_g) @ rx + mag(Wu_bits, s_u) @ rx + mag(Wd_bits, s_d).sum(axis=0) * ra


def select_dense_ref(score: np.ndarray, k: int) -> np.ndarray:
    """The k highest scores, ties to the lower index; returned ascending.

    Infinite scores take their place in the order; a NaN score has none and is
    rejected (ValueError)."""
    score = np.asarray(score, dtype=np.float64)
    if np.any(np.isnan(score)):
        raise ValueError("NaN score")
    order = np.argsort(-score, kind="stable")
    return np.sort(order[:k])


# ---------------------------------------------------------------------------
# W8A8: e4m3 weights times per-token e4m3 activations.  The SpenseGPT
# explainer (Technical Summary 4, "Experimental Results") runs its layers in
# FP8; the SlideSparse explainer (Methodology 2.B "Activation Lifting" and
# 2.C "System integration") quantises activations per token online, folding
# the activation column re-ordering into that same pass, ahead of the 2:4
# sparse GEMM.  Neither page fixes the scale rule; the reading here is the
# plain absmax one:
#     s_x[m] = max_k |X[m, k]| / 448  (fp32 quotient; 448 = largest e4m3fn value),
#              1 for an all-zero row,
#     q[m, k] = the e4m3fn value nearest to the fp32 quotient X[m, k] / s_x[m],
#              ties to the even code (mantissa LSB 0); magnitudes beyond 448
#              saturate to 448; the sign is kept (a negative value that rounds
#              to zero gives -0),
# and the layer output is Y[m, n] = s_x[m] * s[n] * sum_k q[m, k] * Wp[n, k].
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0
# non-negative e4m3fn values, increasing with the code: 0x00 (zero), 0x01..0x07
# (subnormals), 0x08..0x7E (normals); 0x7F is NaN
_E4M3_POS = _E4M3_TABLE[:0x7F]


def e4m3_round(v) -> np.ndarray:
    """float32 values -> e4m3fn codes (uint8), round to nearest, ties to even, saturating."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v.astype(np.float64))
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    code = np.where(d_hi < d_lo, hi, np.where(d_lo < d_hi, lo, np.where(hi % 2 == 0, hi, lo)))
    code = np.where(a >= E4M3_MAX, 0x7E, code)  # at or beyond the largest value (saturation)
    code = code.astype(np.uint8) | np.where(np.signbit(v), np.uint8(0x80), np.uint8(0))
    return np.where(np.isnan(v), np.uint8(0x7F), code).astype(np.uint8)


def quantize_tokens_ref(X_bits: np.ndarray, xdtype: int = DT_BF16):
    """Per-token e4m3 quantisation of X [M, K]: returns (codes uint8 [M, K], s_x float32 [M])."""
    X = decode_values(X_bits, xdtype).astype(np.float32)  # exact for bf16
    amax = np.max(np.abs(X), axis=1) if X.shape[1] else np.zeros(X.shape[0], np.float32)
    sx = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = (X / sx[:, None]).astype(np.float32)  # fp32 quotients
    return e4m3_round(q), sx


def linear_w8a8_ref(codes: np.ndarray, sx: np.ndarray, p: Packed, scales=None):
    """Exact W8A8 layer output in float64 and its error scale.

        Y[m, n] = s_x[m] * s[n] * sum_k q[m, k] * Wp[n, k]
        B[m, n] = s_x[m] * s[n] * sum_k |q[m, k] * Wp[n, k]|
    Products of two e4m3 values carry at most 8 significant bits between 2^-18
    and 2^18, so every partial sum over K < 2^15 terms is exact in float64 and
    the sum does not depend on its order.
    """
    Wp = decompress(p)
    Q = decode_values(codes, DT_FP8)
    acc = Q @ Wp.T
    absacc = np.abs(Q) @ np.abs(Wp).T
    f = np.asarray(sx, dtype=np.float32).astype(np.float64)[:, None]
    if scales is not None:
        f = f * np.asarray(scales, dtype=np.float32).astype(np.float64)[None, :]
    return acc * f, absacc * f
