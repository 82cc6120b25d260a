"""GPU parity of SpenseGPT+ scoring and dense index selection against the oracle.

SpenseGPT explainer, Technical Summary 2.B: score per intermediate index from
|W_ij| sqrt(H_jj) over gate, up and down; the top-scoring indices stay dense.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sparse_dense_gemm_amd as sdg
import synth
from synth import DT_BF16, DT_F32, DT_FP8

from spense_gpu_util import log, to_dev

pytestmark = pytest.mark.gpu


def _block(H, I, T, wdt, seed):
    rng = np.random.default_rng(seed)
    Wgu, sgu = synth.make_weight(2 * I, H, wdt, rng)
    Wd, sd = synth.make_weight(H, I, wdt, rng)
    Xc = synth.make_x(T, H, DT_BF16, rng)
    Ac = synth.make_x(T, I, DT_BF16, rng)
    return Wgu, sgu, Wd, sd, Xc, Ac


def _device_scores(H, I, wdt, Wgu, sgu, Wd, sd, Xc, Ac):
    score = torch.empty(I, dtype=torch.float32, device="cuda")
    sdg.spense_score_glu(to_dev(Wgu, wdt), to_dev(Wd, wdt), wdt, H=H, I=I, X_cal=to_dev(Xc, DT_BF16),
                         A_cal=to_dev(Ac, DT_BF16), score=score,
                         s_gu=None if sgu is None else to_dev(sgu, DT_F32),
                         s_down=None if sd is None else to_dev(sd, DT_F32))
    torch.cuda.synchronize()
    return score


@pytest.mark.parametrize("H,I,T,wdt", [(256, 640, 100, DT_FP8), (132, 388, 64, DT_BF16), (64, 96, 1, DT_FP8)])
def test_scores_and_selection(H, I, T, wdt):
    Wgu, sgu, Wd, sd, Xc, Ac = _block(H, I, T, wdt, 91)
    score = _device_scores(H, I, wdt, Wgu, sgu, Wd, sd, Xc, Ac)
    ref = oracle.glu_scores_ref(Xc, Ac, DT_BF16, Wgu[:I], Wgu[I:], Wd, wdt,
                                None if sgu is None else sgu[:I], None if sgu is None else sgu[I:], sd)
    got = score.cpu().numpy().astype(np.float64)
    # every term is nonnegative: fp32 sums stay within a small relative error
    rel = np.max(np.abs(got - ref) / ref)
    assert rel <= 1e-4, rel
    for k in (0, 1, I // 4, I - 1, I):
        sel = sdg.spense_select_dense(score, k)
        # the decision taken on the device's own fp32 scores is exactly the rank rule
        assert np.array_equal(sel, oracle.select_dense_ref(got, k)), k
        # against the float64 scores: only near-ties may differ
        want = oracle.select_dense_ref(ref, k)
        diff = np.setxor1d(sel, want)
        if diff.size:
            kth = np.sort(ref)[::-1][k - 1]
            assert np.all(np.abs(ref[diff] - kth) <= 1e-4 * kth), (k, diff)
    log(f"[score] H={H} I={I} T={T} wdtype={wdt}: max relative error {rel:.2e}")


def test_selection_ties_go_to_lower_index():
    rng = np.random.default_rng(92)
    for n in (1, 7, 300, 1000):
        sc = rng.integers(0, 5, size=n).astype(np.float32)
        d = torch.from_numpy(sc).cuda()
        for k in sorted({0, 1, n // 3, n // 2, n}):
            assert np.array_equal(sdg.spense_select_dense(d, k), oracle.select_dense_ref(sc.astype(np.float64), k))


def test_selection_with_infinities_and_nan():
    """Infinite scores take their place in the order; a NaN score is rejected
    with SPENSE_EINVAL, like the oracle rejects it."""
    sc = np.array([1.0, np.inf, -np.inf, 2.0, np.inf, 0.0, -np.inf, 3.0], dtype=np.float32)
    d = torch.from_numpy(sc).cuda()
    for k in range(len(sc) + 1):
        assert np.array_equal(sdg.spense_select_dense(d, k), oracle.select_dense_ref(sc.astype(np.float64), k)), k
    sc[5] = np.nan
    with pytest.raises(ValueError):
        oracle.select_dense_ref(sc.astype(np.float64), 3)
    with pytest.raises(sdg.SpenseError) as e:
        sdg.spense_select_dense(torch.from_numpy(sc).cuda(), 3)
    assert e.value.status == sdg.SPENSE_EINVAL


def test_scores_are_repeatable():
    H, I, T, wdt = 128, 256, 130, DT_FP8
    args = _block(H, I, T, wdt, 93)
    a = _device_scores(H, I, wdt, *args)
    b = _device_scores(H, I, wdt, *args)
    assert torch.equal(a, b)


def test_selected_set_feeds_the_block():
    """Scores -> dense set -> packed GLU block: the block runs on the chosen
    set and matches the oracle block on that set."""
    H, I, T, wdt = 256, 512, 64, DT_FP8
    Wgu, sgu, Wd, sd, Xc, Ac = _block(H, I, T, wdt, 94)
    score = _device_scores(H, I, wdt, Wgu, sgu, Wd, sd, Xc, Ac)
    D = sdg.spense_select_dense(score, I // 4)
    h = sdg.spense_pack_glu(to_dev(Wgu, wdt), to_dev(Wd, wdt), wdt, H=H, I=I, s_gu=to_dev(sgu, DT_F32),
                            s_down=to_dev(sd, DT_F32), dense_idx=D)
    try:
        M = 4
        A = torch.empty((M, I), dtype=torch.bfloat16, device="cuda")
        Y = torch.empty((M, H), dtype=torch.float32, device="cuda")
        sdg.spense_glu(h, to_dev(Xc[:M], DT_BF16), A, Y)
        torch.cuda.synchronize()
        r = oracle.glu_block_ref(Xc[:M], DT_BF16, Wgu[:I], Wgu[I:], Wd, wdt, D, sgu[:I], sgu[I:], sd)
        a_nat = np.zeros((M, I))
        a_nat[:, r["rho"]] = A.float().cpu().numpy()
        pi, K_s, _ = oracle.resolve_dense_set(I, dense_cols=D)
        Yref, B = oracle.down_ref(a_nat, oracle.pack(Wd, wdt, pi, K_s), sd)
        assert np.all(np.abs(Y.cpu().numpy() - Yref) <= 1e-3 * B)
    finally:
        sdg.spense_free(h)
