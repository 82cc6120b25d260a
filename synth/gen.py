"""Seeded draws and storage encodings for synthetic Spense workloads.

Recipe (shared by every workload):
  * weights  W ~ N(0, 0.02) in float64, activations X ~ N(0, 1) in float64,
    drawn from NumPy's PCG64 ``default_rng(seed)`` in row-major order;
  * fp32 storage: float64 -> float32, round to nearest even;
  * bf16 storage: float64 -> float32 -> bfloat16, each step round to nearest
    even (the bf16 step keeps the top 16 bits after RNE on the low 16);
  * fp8 storage: OCP e4m3fn (bias 7, largest finite 448, no infinities) with a
    per-output-channel float32 scale s[n] = max_k |W[n,k]| / 448; the stored
    code is the e4m3 value nearest to W[n,k] / s[n] (ties to even, saturating
    at 448);
  * dense-column sets: either the contiguous tail of K, or the first K_d
    entries of ``default_rng(seed).permutation(K)``, sorted ascending.

Storage arrays: fp32 -> ``np.float32``; bf16 -> ``np.uint16`` bit patterns;
fp8 -> ``np.uint8`` codes.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# dtype tags; the numbering is the one the C interface uses
DT_F32 = 0
DT_BF16 = 1
DT_FP8 = 2

_ROW_CHUNK = 2048


def bf16_encode(x) -> np.ndarray:
    """float64/float32 array -> bfloat16 bit patterns (uint16), RNE via float32."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def e4m3_encode(x) -> np.ndarray:
    """float array -> OCP e4m3fn codes (uint8): round to nearest even, saturate at 448.

    Exact on the float64 bit pattern.  For |x| >= 2^-6 (normal e4m3) the 52-bit
    fraction is rounded to 3 bits (ties to even) by integer addition, the
    carry stepping into the exponent when the fraction rounds up; the biased
    float64 exponent then maps to the e4m3 exponent by subtracting 1023 - 7.
    Below 2^-6 the subnormal code is rint(|x| * 2^9).
    """
    a = np.minimum(np.abs(np.asarray(x, dtype=np.float64)), 448.0)
    sign = (np.signbit(np.asarray(x, dtype=np.float64)).astype(np.uint8) << 7).astype(np.uint8)
    u = a.view(np.uint64)
    lsb = (u >> np.uint64(49)) & np.uint64(1)
    rounded = (u + np.uint64((1 << 48) - 1) + lsb) >> np.uint64(49)
    normal = a >= 2.0 ** -6
    code_n = rounded.astype(np.int64) - ((1023 - 7) << 3)
    code_s = np.rint(a * 512.0).astype(np.int64)
    code = np.where(normal, code_n, code_s)
    return np.minimum(code, 0x7E).astype(np.uint8) | sign


def _draw_normal(rng: np.random.Generator, rows: int, cols: int, std: float) -> np.ndarray:
    return rng.normal(0.0, std, size=(rows, cols))


def _encode_rows(w: np.ndarray, dtype: int, out: np.ndarray, scales, r0: int, r1: int) -> None:
    if dtype == DT_F32:
        out[r0:r1] = w.astype(np.float32)
    elif dtype == DT_BF16:
        out[r0:r1] = bf16_encode(w)
    else:
        s = (np.max(np.abs(w), axis=1) / 448.0).astype(np.float32)
        s = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
        scales[r0:r1] = s
        out[r0:r1] = e4m3_encode(w / s.astype(np.float64)[:, None])


def make_weight(N: int, K: int, dtype: int, rng: np.random.Generator):
    """Draw W[N,K] ~ N(0, 0.02) and encode it.  Returns (bits, scales-or-None).

    Rows are drawn in chunks, in order, from the one generator (PCG64 normal
    draws fill row-major, so the result equals one (N, K) draw); the encoding
    of finished chunks runs on worker threads while later chunks are drawn.
    """
    if dtype == DT_F32:
        out = np.empty((N, K), np.float32)
    elif dtype == DT_BF16:
        out = np.empty((N, K), np.uint16)
    elif dtype == DT_FP8:
        out = np.empty((N, K), np.uint8)
    else:
        raise ValueError(f"unknown dtype {dtype}")
    scales = np.empty((N,), np.float32) if dtype == DT_FP8 else None
    workers = max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        futs = []
        for r0 in range(0, N, _ROW_CHUNK):
            r1 = min(N, r0 + _ROW_CHUNK)
            w = _draw_normal(rng, r1 - r0, K, 0.02)
            futs.append(pool.submit(_encode_rows, w, dtype, out, scales, r0, r1))
            # bound the number of drawn-but-unencoded chunks held in memory
            while len(futs) > 2 * workers:
                futs.pop(0).result()
        for f in futs:
            f.result()
    return out, scales


def make_x(M: int, K: int, dtype: int, rng: np.random.Generator) -> np.ndarray:
    """Draw X[M,K] ~ N(0, 1): fp32 -> float32 array, bf16 -> uint16 bits."""
    x = _draw_normal(rng, M, K, 1.0)
    if dtype == DT_F32:
        return x.astype(np.float32)
    if dtype == DT_BF16:
        return bf16_encode(x)
    raise ValueError(f"activation dtype {dtype} not drawn")


def tail_dense_set(K: int, K_d: int) -> np.ndarray:
    return np.arange(K - K_d, K, dtype=np.int32)


def random_dense_set(K: int, K_d: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return np.sort(rng.permutation(K)[:K_d]).astype(np.int32)
