"""Helpers shared by the GPU tests: move synth inputs to the device, run the
HIP library through its C interface, fetch its canonical export, and compare
with the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import sparse_dense_gemm_amd as sdg
from synth import DT_BF16, DT_F32, DT_FP8

TOL = 1e-3  # |Y - Y_ref| <= TOL * sum_k |x_k w_k|, per element, fp32 output


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: int) -> torch.Tensor:
    if dtype == DT_F32:
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    if dtype == DT_BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def storage_torch_dtype(dtype: int):
    return {DT_F32: torch.float32, DT_BF16: torch.int16, DT_FP8: torch.uint8}[dtype]


def pack_dev(Wd: torch.Tensor, dtype: int, scales_d, dense_cols=None, dense_fraction=0.0) -> int:
    return sdg.spense_pack(Wd, dtype, scales=scales_d, dense_cols=dense_cols, dense_fraction=dense_fraction)


def export(h: int, dtype: int, rows=None):
    """Canonical packed form from the device; optionally only the given rows (numpy)."""
    info = sdg.spense_info(h)
    N, K_s, K_d = info["N"], info["K_s"], info["K_d"]
    mw = (K_s // 4 + 7) // 8
    sd = storage_torch_dtype(dtype)
    vals = torch.empty((N, K_s // 2), dtype=sd, device="cuda")
    meta = torch.empty((N, mw), dtype=torch.int32, device="cuda")
    mask = torch.empty((N, K_s), dtype=torch.uint8, device="cuda")
    dense = torch.empty((N, K_d), dtype=sd, device="cuda")
    pi = sdg.spense_export(h, vals, meta, mask, dense)
    if rows is not None:
        r = torch.as_tensor(rows, device="cuda", dtype=torch.long)
        vals, meta, mask, dense = vals[r], meta[r], mask[r], dense[r]
    out = dict(vals=vals.cpu().numpy(), meta=meta.cpu().numpy().view(np.uint32), mask=mask.cpu().numpy(),
               dense=dense.cpu().numpy(), pi=pi)
    if dtype == DT_BF16:
        out["vals"] = out["vals"].view(np.uint16)
        out["dense"] = out["dense"].view(np.uint16)
    return out


def assert_pack_equal(got: dict, ref: oracle.Packed):
    assert np.array_equal(got["pi"], ref.pi.astype(np.int32)), "pi"
    assert np.array_equal(got["mask"], ref.mask), "mask"
    assert np.array_equal(got["meta"], ref.meta), "meta"
    assert np.array_equal(got["vals"].view(np.uint8), np.ascontiguousarray(ref.vals).view(np.uint8)), "vals"
    assert np.array_equal(got["dense"].view(np.uint8), np.ascontiguousarray(ref.dense).view(np.uint8)), "dense"


def linear_dev(h: int, Xd: torch.Tensor, N: int, ydtype: int = DT_F32, splits: int = 0, M=None) -> torch.Tensor:
    M = Xd.shape[0] if M is None else M
    Y = torch.empty((M, N), dtype=torch.float32 if ydtype == DT_F32 else torch.bfloat16, device="cuda")
    sdg.spense_linear_splits(h, Xd, Y, splits, M=M)
    torch.cuda.synchronize()
    return Y


def tol_ratio(Y: np.ndarray, Yref: np.ndarray, B: np.ndarray) -> float:
    """max |Y - Yref| / (TOL * B); <= 1 passes.  Entries with B == 0 must match exactly."""
    err = np.abs(Y.astype(np.float64) - Yref)
    zero = B == 0
    assert np.all(err[zero] == 0), "nonzero output where every product is zero"
    if np.all(zero):
        return 0.0
    return float(np.max(err[~zero] / (TOL * B[~zero])))


def oracle_pack_rows(W: np.ndarray, dtype: int, D, rows=None):
    pi, K_s, K_d = oracle.resolve_dense_set(W.shape[1], dense_cols=D)
    Wr = W if rows is None else W[rows]
    return oracle.pack(Wr, dtype, pi, K_s)
