"""GPU parity of the output-split layer (spense_pack_rows) against the oracle.

Output-split form, SpenseGPT explainer Technical Summary 2.A: dense rows keep
every weight, the other rows are 2:4 along K; the row classes write different
output columns.  Every call goes through the C interface.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sparse_dense_gemm_amd as sdg
import synth
from synth import DT_BF16, DT_F32, DT_FP8

from spense_gpu_util import linear_dev, log, storage_torch_dtype, to_dev, tol_ratio

pytestmark = pytest.mark.gpu


def _weights(N, K, wdtype, seed):
    W, s = synth.make_weight(N, K, wdtype, np.random.default_rng(seed))
    return W, s


def _pack_rows_dev(W, s, wdtype, dense_rows=None, dense_fraction=0.0):
    sd = to_dev(s, DT_F32) if s is not None else None
    return sdg.spense_pack_rows(to_dev(W, wdtype), wdtype, scales=sd, dense_rows=dense_rows,
                                dense_fraction=dense_fraction)


def _export_rows(h, wdtype):
    info = sdg.spense_info(h)
    N, K, N_s, N_d = info["N"], info["K"], info["N_s"], info["N_d"]
    sd = storage_torch_dtype(wdtype)
    vals = torch.empty((N_s, K // 2), dtype=sd, device="cuda")
    meta = torch.empty((N_s, (K // 4 + 7) // 8), dtype=torch.int32, device="cuda")
    mask = torch.empty((N_s, K), dtype=torch.uint8, device="cuda")
    dense = torch.empty((N_d, K), dtype=sd, device="cuda")
    rho = sdg.spense_export_rows(h, vals, meta, mask, dense)
    return dict(rho=rho, vals=vals.cpu().numpy().view(np.uint8), meta=meta.cpu().numpy().view(np.uint32),
                mask=mask.cpu().numpy(), dense=dense.cpu().numpy().view(np.uint8))


def _oracle_rows(W, wdtype, dense_rows=None, dense_fraction=None):
    N, K = W.shape
    rho, N_s, _ = oracle.resolve_dense_rows(N, K, dense_rows=dense_rows, dense_fraction=dense_fraction)
    return oracle.pack_rows(W, wdtype, rho, N_s)


CASES = [
    # (N, K, wdtype, dense rows: ("frac", p) or ("rand", count))
    (200, 512, DT_FP8, ("frac", 0.25)),
    (200, 512, DT_BF16, ("rand", 37)),
    (77, 388, DT_FP8, ("rand", 20)),      # ragged N and K (K % 128 != 0: padded, gathered)
    (96, 256, DT_FP8, ("frac", 0.0)),     # no dense row
    (96, 256, DT_BF16, ("frac", 1.0)),    # no sparse row
    (33, 128, DT_FP8, ("rand", 1)),
]


def _dense_arg(N, spec, seed):
    if spec[0] == "frac":
        return dict(dense_fraction=spec[1]), dict(dense_fraction=spec[1])
    D = synth.random_dense_set(N, spec[1], seed)
    return dict(dense_rows=D), dict(dense_rows=D)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"N{c[0]}K{c[1]}w{c[2]}{c[3][0]}{c[3][1]}")
def test_export_rows_bit_exact(case):
    N, K, wdt, spec = case
    W, s = _weights(N, K, wdt, 61)
    dev_kw, ora_kw = _dense_arg(N, spec, 62)
    h = _pack_rows_dev(W, s, wdt, **dev_kw)
    try:
        got = _export_rows(h, wdt)
        ref = _oracle_rows(W, wdt, **ora_kw)
        info = sdg.spense_info(h)
        assert info["split"] == 1 and info["N_s"] == ref.N_s and info["N_d"] == ref.N_d
        b = 1 if wdt == DT_FP8 else 2
        assert info["weight_bytes"] == ref.N_s * (K // 2 * b + K // 8) + ref.N_d * K * b
        assert np.array_equal(got["rho"], ref.rho.astype(np.int32))
        if ref.N_s:
            assert np.array_equal(got["mask"], ref.sparse.mask)
            assert np.array_equal(got["meta"], ref.sparse.meta)
            assert np.array_equal(got["vals"], np.ascontiguousarray(ref.sparse.vals).view(np.uint8))
        if ref.N_d:
            assert np.array_equal(got["dense"], np.ascontiguousarray(ref.dense).view(np.uint8))
        log(f"[output-split export] N={N} K={K} wdtype={wdt} {spec}: bit-exact")
    finally:
        sdg.spense_free(h)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"N{c[0]}K{c[1]}w{c[2]}{c[3][0]}{c[3][1]}")
def test_linear_rows_within_tolerance(case):
    N, K, wdt, spec = case
    W, s = _weights(N, K, wdt, 63)
    X = synth.make_x(130, K, DT_BF16, np.random.default_rng(64))
    dev_kw, ora_kw = _dense_arg(N, spec, 65)
    h = _pack_rows_dev(W, s, wdt, **dev_kw)
    try:
        ref = _oracle_rows(W, wdt, **ora_kw)
        Xd = to_dev(X, DT_BF16)
        worst = 0.0
        for M in (1, 5, 16, 17, 64, 130):
            Yref, B = oracle.linear_rows_ref(X[:M], DT_BF16, ref, s)
            for sp in ((0, 1, 2) if K >= 256 else (0, 1)):
                Y = linear_dev(h, Xd[:M], N, splits=sp).cpu().numpy()
                r = tol_ratio(Y, Yref, B)
                assert r <= 1.0, (M, sp, r)
                worst = max(worst, r)
        log(f"[output-split linear] N={N} K={K} wdtype={wdt} {spec}: worst error {worst:.2e} of tolerance")
    finally:
        sdg.spense_free(h)


def test_row_classes_match_single_class_layers_bitwise():
    """With one split, the 2:4 rows of an output-split layer give bitwise the
    outputs of an input-split layer with no dense columns, and the dense rows
    those of the all-dense layer (same kernels, same accumulation order)."""
    N, K, M = 160, 1024, 7
    W, s = _weights(N, K, DT_FP8, 66)
    X = synth.make_x(M, K, DT_BF16, np.random.default_rng(67))
    D = synth.random_dense_set(N, 40, 68)
    dense = np.zeros(N, dtype=bool)
    dense[D] = True
    sd = to_dev(s, DT_F32)
    Wd = to_dev(W, DT_FP8)
    h = sdg.spense_pack_rows(Wd, DT_FP8, scales=sd, dense_rows=D)
    h_sp = sdg.spense_pack(Wd, DT_FP8, scales=sd, dense_fraction=0.0)
    h_de = sdg.spense_pack(Wd, DT_FP8, scales=sd, dense_fraction=1.0)
    try:
        Xd = to_dev(X, DT_BF16)
        Y = linear_dev(h, Xd, N, splits=1).cpu().numpy()
        Ysp = linear_dev(h_sp, Xd, N, splits=1).cpu().numpy()
        Yde = linear_dev(h_de, Xd, N, splits=1).cpu().numpy()
        assert np.array_equal(Y[:, ~dense], Ysp[:, ~dense])
        assert np.array_equal(Y[:, dense], Yde[:, dense])
        log("[output-split] row classes bitwise equal to the single-class layers")
    finally:
        for hh in (h, h_sp, h_de):
            sdg.spense_free(hh)


def test_rows_bf16_output_is_rne_of_fp32():
    N, K, M = 64, 256, 4
    W, s = _weights(N, K, DT_FP8, 69)
    X = synth.make_x(M, K, DT_BF16, np.random.default_rng(70))
    h = _pack_rows_dev(W, s, DT_FP8, dense_fraction=0.25)
    try:
        Xd = to_dev(X, DT_BF16)
        Y32 = linear_dev(h, Xd, N, ydtype=DT_F32, splits=1)
        Y16 = linear_dev(h, Xd, N, ydtype=DT_BF16, splits=1)
        assert torch.equal(Y32.to(torch.bfloat16), Y16)
    finally:
        sdg.spense_free(h)
