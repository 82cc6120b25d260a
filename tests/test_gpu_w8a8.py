"""GPU parity of the W8A8 form (spense_quantize_tokens, spense_linear_w8a8)
against the oracle.

SpenseGPT explainer, Technical Summary 4 (layers in FP8) with the SlideSparse
explainer's Methodology 2.B/2.C (per-token activation quantisation online,
the column re-ordering folded into it).  The codes are an integer decision
taken in fp32 on both sides (absmax / 448, fp32 quotient, round to nearest
even), so they must match bit for bit; the layer output must lie within
1e-3 * sum |q_x q_w| * s_x * s of the exact result.
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

TILE_PRESETS = list(range(17))


def _quantize_dev(X: np.ndarray):
    M, K = X.shape
    Xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    sdg.spense_quantize_tokens(to_dev(X, DT_BF16), Xq, sx)
    torch.cuda.synchronize()
    return Xq.cpu().numpy(), sx.cpu().numpy()


def _tie_rows(K, rng):
    """Tokens whose scale is exactly 1 (largest magnitude 448) and whose other
    values sit on e4m3 midpoints, so every code is a round-half-even decision."""
    pos = oracle.decode_values(np.arange(0x7F, dtype=np.uint8), DT_FP8)
    mids = (pos[1:] + pos[:-1]) / 2
    v = rng.choice(mids, size=(2, K)) * rng.choice([-1.0, 1.0], size=(2, K))
    v[:, 0] = 448.0
    return torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.uint16).numpy()


@pytest.mark.parametrize("M,K", [(1, 64), (7, 300), (130, 5120), (3, 13)])
def test_quantize_tokens_bit_exact(M, K):
    rng = np.random.default_rng(500 + K)
    X = synth.make_x(M, K, DT_BF16, rng)
    if M >= 7:
        X[2] = 0                       # all-zero token: scale 1, codes 0
        X[3] = _tie_rows(K, rng)[0]    # ties
        X[4] = (X[4].astype(np.uint32) & 0x7FFF).astype(np.uint16) | 0x8000  # all negative
    q, sx = _quantize_dev(X)
    q_ref, sx_ref = oracle.quantize_tokens_ref(X, DT_BF16)
    assert np.array_equal(sx.view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(q, q_ref)
    log(f"[w8a8 quantize] M={M} K={K}: codes and scales bit-exact")


CASES = [
    # (N, K, dense spec)
    (200, 512, ("frac", 0.25)),
    (77, 388, ("rand", 20)),       # ragged N and K, chosen set (re-ordered while quantising)
    (96, 256, ("frac", 0.0)),      # pure 2:4
    (96, 256, ("frac", 1.0)),      # all dense
    (50, 200, ("frac", 0.26)),     # K_s = 148: padded steps
    (33, 128, ("rand", 4)),
]


def _pack_case(N, K, dense, seed):
    W, s = synth.make_weight(N, K, DT_FP8, np.random.default_rng(seed))
    sd = to_dev(s, DT_F32)
    if dense[0] == "frac":
        pi, K_s, _ = oracle.resolve_dense_set(K, dense_fraction=dense[1])
        D = np.sort(pi[K_s:])
        h = pack_dev(to_dev(W, DT_FP8), DT_FP8, sd, dense_fraction=dense[1])
    else:
        D = synth.random_dense_set(K, dense[1], seed + 1)
        h = pack_dev(to_dev(W, DT_FP8), DT_FP8, sd, dense_cols=D)
    return W, s, D, h


def _w8a8_dev(h, Xd, N, ydtype=DT_F32, splits=0):
    Y = torch.empty((Xd.shape[0], N), dtype=torch.float32 if ydtype == DT_F32 else torch.bfloat16, device="cuda")
    sdg.spense_linear_w8a8(h, Xd, Y, splits=splits)
    torch.cuda.synchronize()
    return Y


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"N{c[0]}K{c[1]}{c[2][0]}{c[2][1]}")
def test_linear_w8a8_within_tolerance(case):
    N, K, dense = case
    W, s, D, h = _pack_case(N, K, dense, 510 + N)
    try:
        ref = oracle_pack_rows(W, DT_FP8, D)
        X = synth.make_x(130, K, DT_BF16, np.random.default_rng(520 + K))
        Xd = to_dev(X, DT_BF16)
        worst = 0.0
        for M in (1, 5, 16, 17, 64, 130):
            q, sx = oracle.quantize_tokens_ref(X[:M], DT_BF16)
            Yref, B = oracle.linear_w8a8_ref(q, sx, ref, s)
            for sp in ((0, 1, 2) if K >= 256 else (0, 1)):
                Y = _w8a8_dev(h, Xd[:M], N, splits=sp).cpu().numpy()
                r = tol_ratio(Y, Yref, B)
                assert r <= 1.0, (M, sp, r)
                worst = max(worst, r)
        log(f"[w8a8 linear] N={N} K={K} {dense}: worst error {worst:.2e} of tolerance")
    finally:
        sdg.spense_free(h)


@pytest.mark.parametrize("dense", [("frac", 0.25), ("rand", 192)])
def test_w8a8_tile_presets(dense, monkeypatch):
    """Every register-blocked configuration of the W8A8 streaming kernel on
    ragged row counts, batches ending mid m-tile and several split counts."""
    N, K = 232, 1536
    W, s, D, h = _pack_case(N, K, dense, 530)
    try:
        ref = oracle_pack_rows(W, DT_FP8, D)
        X = synth.make_x(130, K, DT_BF16, np.random.default_rng(531))
        Xd = to_dev(X, DT_BF16)
        for M in (17, 40, 64, 130):
            q, sx = oracle.quantize_tokens_ref(X[:M], DT_BF16)
            Yref, B = oracle.linear_w8a8_ref(q, sx, ref, s)
            for v in TILE_PRESETS:
                monkeypatch.setenv("SPENSE_TILE", str(v))
                for sp in (0, 1, 3):
                    Y = _w8a8_dev(h, Xd[:M], N, splits=sp).cpu().numpy()
                    r = tol_ratio(Y, Yref, B)
                    assert r <= 1.0, (v, M, sp, r)
        log(f"[w8a8 tile presets] dense={dense}: all presets within tolerance")
    finally:
        sdg.spense_free(h)


@pytest.mark.parametrize("dense", [("frac", 0.25), ("rand", 192)])
def test_w8a8_lds_tile_presets(dense, monkeypatch):
    """Every configuration of the LDS-staged kernel on e4m3 activation codes:
    ragged row counts, batches ending mid m-tile, several m-groups and split counts."""
    N, K = 232, 1536
    W, s, D, h = _pack_case(N, K, dense, 532)
    try:
        ref = oracle_pack_rows(W, DT_FP8, D)
        X = synth.make_x(300, K, DT_BF16, np.random.default_rng(533))
        Xd = to_dev(X, DT_BF16)
        for M in (17, 40, 64, 130, 300):
            q, sx = oracle.quantize_tokens_ref(X[:M], DT_BF16)
            Yref, B = oracle.linear_w8a8_ref(q, sx, ref, s)
            for v in range(8):
                monkeypatch.setenv("SPENSE_LDS", str(v))
                for sp in (0, 1, 3):
                    Y = _w8a8_dev(h, Xd[:M], N, splits=sp).cpu().numpy()
                    r = tol_ratio(Y, Yref, B)
                    assert r <= 1.0, (v, M, sp, r)
        log(f"[w8a8 lds presets] dense={dense}: all configurations within tolerance")
    finally:
        sdg.spense_free(h)


def test_w8a8_bf16_output_repeatable_and_rne():
    N, K, M = 160, 1024, 48
    W, s, D, h = _pack_case(N, K, ("rand", 256), 540)
    try:
        Xd = to_dev(synth.make_x(M, K, DT_BF16, np.random.default_rng(541)), DT_BF16)
        y1 = _w8a8_dev(h, Xd, N, splits=3)
        y2 = _w8a8_dev(h, Xd, N, splits=3)
        assert torch.equal(y1, y2)
        yb = _w8a8_dev(h, Xd, N, ydtype=DT_BF16, splits=3)
        assert torch.equal(y1.to(torch.bfloat16), yb)
    finally:
        sdg.spense_free(h)


def test_w8a8_rejects_other_layers():
    W, s = synth.make_weight(64, 256, DT_BF16, np.random.default_rng(550))
    h = pack_dev(to_dev(W, DT_BF16), DT_BF16, None, dense_fraction=0.25)
    try:
        Xd = to_dev(synth.make_x(4, 256, DT_BF16, np.random.default_rng(551)), DT_BF16)
        Y = torch.empty((4, 64), dtype=torch.float32, device="cuda")
        with pytest.raises(RuntimeError):
            sdg.spense_linear_w8a8(h, Xd, Y)
    finally:
        sdg.spense_free(h)


def _sample_rows(N):
    NT = (N + 15) // 16
    tiles = np.unique(np.concatenate([np.linspace(0, NT - 1, 24).astype(np.int64), [0, NT - 1]]))
    return np.concatenate([np.arange(16 * t, min(N, 16 * t + 16)) for t in tiles])


@pytest.mark.parametrize("lname", [s.name for s in synth.WORKLOADS["layer36b_fp8"].layers])
def test_w8a8_full_layer_sampled(lname):
    """The 36B-class layers at their real shapes and batches (128 and 2048
    tokens; 2048 is the launch configuration the benchmark times): a spread
    sample of row tiles for a sample of tokens, against the exact W8A8 result."""
    w = synth.WORKLOADS["layer36b_fp8"]
    spec = next(x for x in w.layers if x.name == lname)
    M = max(w.Ms)
    W, s, X, D = synth.layer_inputs(spec, M)
    h = pack_dev(to_dev(W, DT_FP8), DT_FP8, to_dev(s, DT_F32), dense_cols=D)
    try:
        Xd = to_dev(X, DT_BF16)
        rows = _sample_rows(spec.N)
        ref = oracle_pack_rows(W, DT_FP8, D, rows)
        for Mc in w.Ms:
            sel = np.unique(np.concatenate([np.random.default_rng(552 + Mc).choice(Mc, 30, replace=False), [0, Mc - 1]]))
            # a token's codes depend on that token alone
            q, sx = oracle.quantize_tokens_ref(X[sel], DT_BF16)
            Yref, B = oracle.linear_w8a8_ref(q, sx, ref, s[rows])
            Y = _w8a8_dev(h, Xd[:Mc], spec.N).cpu().numpy()
            r = tol_ratio(Y[sel][:, rows], Yref, B)
            log(f"[w8a8 full] {lname} N={spec.N} K={spec.K} M={Mc}: ratio {r:.3e} on {sel.size} tokens x {rows.size} rows")
            assert r <= 1.0
    finally:
        sdg.spense_free(h)


def test_leading_dimensions_beyond_32bit_offsets_are_refused():
    """The streaming kernels address staged activations with 32-bit offsets:
    a leading dimension of 2^23 elements or more is refused on the host
    (M = 1, so even a kernel launch would read only row 0, which exists)."""
    N, K = 64, 256
    W, s = synth.make_weight(N, K, DT_FP8, np.random.default_rng(560))
    h = pack_dev(to_dev(W, DT_FP8), DT_FP8, to_dev(s, DT_F32), dense_fraction=0.25)
    try:
        Xd = to_dev(synth.make_x(1, K, DT_BF16, np.random.default_rng(561)), DT_BF16)
        Y = torch.empty((1, N), dtype=torch.float32, device="cuda")
        with pytest.raises(sdg.SpenseError) as e:
            sdg.spense_linear_splits(h, Xd, Y, 0, ldx=1 << 23)
        assert e.value.status == sdg.SPENSE_EUNSUPPORTED
        Y1 = torch.empty_like(Y)
        sdg.spense_linear_splits(h, Xd, Y1, 0, ldx=(1 << 23) - 1)  # just below the limit: accepted
        sdg.spense_linear_splits(h, Xd, Y, 0)
        torch.cuda.synchronize()
        assert torch.equal(Y, Y1)
        # the W8A8 path reads the caller's rows only in its quantisation pass
        # (64-bit offsets) and stages its own workspace: any leading dimension works
        sdg.spense_linear_w8a8(h, Xd, Y1, ldx=1 << 23)
        sdg.spense_linear_w8a8(h, Xd, Y)
        torch.cuda.synchronize()
        assert torch.equal(Y, Y1)
    finally:
        sdg.spense_free(h)
