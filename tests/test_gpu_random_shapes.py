"""Seeded random shapes through the planner's own choices (kernel, tile
preset, split count), W8A16 and W8A8, against the oracle.

The parity rule is the layer tolerance of the Spense linear layer (SpenseGPT
explainer, Technical Summary 2.A: sparse product plus dense product into one
output); the shapes cover ragged row tiles, 2:4 regions that end inside a
128-column step, tail and chosen dense sets, and batch sizes on both sides of
every planner threshold.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sparse_dense_gemm_amd as sdg
import synth
from synth import DT_BF16, DT_F32, DT_FP8

from spense_gpu_util import log, oracle_pack_rows, pack_dev, to_dev, tol_ratio

pytestmark = pytest.mark.gpu


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    N = int(rng.integers(17, 720))
    K = int(rng.integers(16, 520)) * 4
    M = int(rng.choice([1, 3, 7, 16, 17, 33, 64, 65, 130, 257, 300]))
    if rng.random() < 0.5:
        K_d = int(rng.integers(0, K // 4 + 1)) * 4 if rng.random() < 0.8 else K
        dense = ("rand", K_d)
    else:
        dense = ("frac", float(rng.choice([0.0, 0.125, 0.25, 0.5])))
        K = max(32, K // 32 * 32)  # the fraction then gives whole 2:4 groups
    wdt = DT_FP8 if rng.random() < 0.7 else DT_BF16
    return N, K, M, dense, wdt


@pytest.mark.parametrize("seed", range(14))
def test_random_shape(seed):
    N, K, M, dense, wdt = _case(seed)
    rng = np.random.default_rng(2000 + seed)
    W, s = synth.make_weight(N, K, wdt, rng)
    X = synth.make_x(M, K, DT_BF16, rng)
    sd = to_dev(s, DT_F32) if s is not None else None
    if dense[0] == "frac":
        pi, K_s, _ = oracle.resolve_dense_set(K, dense_fraction=dense[1])
        D = np.sort(pi[K_s:])
        h = pack_dev(to_dev(W, wdt), wdt, sd, dense_fraction=dense[1])
    else:
        D = synth.random_dense_set(K, dense[1], 3000 + seed)
        h = pack_dev(to_dev(W, wdt), wdt, sd, dense_cols=D)
    try:
        ref = oracle_pack_rows(W, wdt, D)
        Xd = to_dev(X, DT_BF16)
        Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        sdg.spense_linear(h, Xd, Y)
        torch.cuda.synchronize()
        Yref, B = oracle.linear_ref(X, DT_BF16, ref, s)
        r = tol_ratio(Y.cpu().numpy(), Yref, B)
        assert r <= 1.0, r
        msg = f"[random {seed}] N={N} K={K} M={M} dense={dense} wdtype={wdt}: W8A16 {r:.2e}"
        if wdt == DT_FP8:
            sdg.spense_linear_w8a8(h, Xd, Y)
            torch.cuda.synchronize()
            q, sx = oracle.quantize_tokens_ref(X, DT_BF16)
            Yref8, B8 = oracle.linear_w8a8_ref(q, sx, ref, s)
            r8 = tol_ratio(Y.cpu().numpy(), Yref8, B8)
            assert r8 <= 1.0, r8
            msg += f", W8A8 {r8:.2e}"
        log(msg + " of tolerance")
    finally:
        sdg.spense_free(h)
