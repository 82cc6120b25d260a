"""Parity of the HIP library (called through its C interface) with the oracle
on small and edge shapes, every kernel variant and launch configuration.

* spense_pack: canonical export equals the oracle's packed form bit for bit.
* spense_linear: every element within 1e-3 * sum_k |x_k w_k| of the oracle's
  float64 result, compared on the fp32 output before any cast.
The benchmark's workloads at their full sizes are in test_gpu_full_size.py.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_dense_gemm_amd as sdg
import synth
from synth import DT_BF16, DT_F32, DT_FP8

from spense_gpu_util import (assert_pack_equal, export, linear_dev, log, oracle_pack_rows, pack_dev, to_dev,
                             tol_ratio)

pytestmark = pytest.mark.gpu

# ---------------------------------------------------------------------------
# edge cases on small shapes
# ---------------------------------------------------------------------------
def _small(N, K, wdtype, seed):
    rng = np.random.default_rng(seed)
    W, s = synth.make_weight(N, K, wdtype, rng)
    return W, s


EDGE = [
    # (N, K, wdtype, dense spec, Ms, splits)
    (50, 200, DT_FP8, ("frac", 0.26), (1, 3, 17), (0, 1, 2)),       # ragged rows, K_s = 148 (not 128-aligned)
    (64, 384, DT_FP8, ("rand", 96), (1, 16, 33, 65), (0, 1, 3)),   # gather path, several m-tiles
    (48, 256, DT_BF16, ("frac", 0.25), (2, 31, 64, 100), (0, 1, 2)),
    (40, 320, DT_BF16, ("rand", 80), (5,), (0, 2)),
    (32, 256, DT_FP8, ("frac", 0.0), (1, 8), (0, 2)),                # pure 2:4
    (32, 256, DT_FP8, ("frac", 1.0), (1, 8), (0, 2)),                # all dense (baseline form)
    (24, 64, DT_BF16, ("frac", 0.5), (1, 7), (0, 1)),                # one macro-step each
    (17, 512, DT_F32, ("frac", 0.25), (1, 4), (0,)),                 # fp32 path
    (33, 100, DT_F32, ("rand", 20), (3,), (0,)),
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: f"N{c[0]}K{c[1]}dt{c[2]}{c[3][0]}{c[3][1]}")
def test_edge_shapes(case):
    N, K, wdtype, dense, Ms, splits_list = case
    log(f"[edge] {case}")
    W, s = _small(N, K, wdtype, 100 + N)
    xdt = DT_F32 if wdtype == DT_F32 else DT_BF16
    X = synth.make_x(max(Ms), K, xdt, np.random.default_rng(200 + K))
    if dense[0] == "frac":
        pi, K_s, K_d = oracle.resolve_dense_set(K, dense_fraction=dense[1])
        D = np.sort(pi[K_s:])
        h = pack_dev(to_dev(W, wdtype), wdtype, to_dev(s, DT_F32) if s is not None else None, dense_fraction=dense[1])
    else:
        D = synth.random_dense_set(K, dense[1], 300 + K)
        h = pack_dev(to_dev(W, wdtype), wdtype, to_dev(s, DT_F32) if s is not None else None, dense_cols=D)
    try:
        ref = oracle_pack_rows(W, wdtype, D)
        assert_pack_equal(export(h, wdtype), ref)
        Xd = to_dev(X, xdt)
        for M in Ms:
            Yref, B = oracle.linear_ref(X[:M], xdt, ref, s)
            for sp in splits_list:
                Y = linear_dev(h, Xd[:M], N, splits=sp).cpu().numpy()
                r = tol_ratio(Y, Yref, B)
                log(f"  M={M} splits={sp}: ratio {r:.3e}")
                assert r <= 1.0
    finally:
        sdg.spense_free(h)


@pytest.mark.parametrize("wdtype", [DT_FP8, DT_BF16])
def test_bf16_output_is_rne_of_fp32_output(wdtype):
    N, K, M = 64, 512, 5
    W, s = _small(N, K, wdtype, 7)
    X = synth.make_x(M, K, DT_BF16, np.random.default_rng(8))
    h = pack_dev(to_dev(W, wdtype), wdtype, to_dev(s, DT_F32) if s is not None else None, dense_fraction=0.25)
    try:
        Xd = to_dev(X, DT_BF16)
        for sp in (1, 3):
            y32 = linear_dev(h, Xd, N, DT_F32, splits=sp)
            y16 = linear_dev(h, Xd, N, DT_BF16, splits=sp)
            assert torch.equal(y32.to(torch.bfloat16).view(torch.int16), y16.view(torch.int16))
    finally:
        sdg.spense_free(h)


@pytest.mark.parametrize("wdtype", [DT_FP8, DT_BF16])
def test_one_hot_rows_are_exact(wdtype):
    """X = rows of the identity: each output is one product, so the result is
    s[n] * Wp[n, k] rounded once to fp32, bit for bit."""
    N, K = 48, 256
    W, s = _small(N, K, wdtype, 9)
    D = synth.random_dense_set(K, 64, 10)
    X = synth.bf16_encode(np.eye(K))
    h = pack_dev(to_dev(W, wdtype), wdtype, to_dev(s, DT_F32) if s is not None else None, dense_cols=D)
    try:
        ref = oracle_pack_rows(W, wdtype, D)
        Wp = oracle.decompress(ref)
        expect = (Wp.T * (s.astype(np.float64)[None, :] if s is not None else 1.0)).astype(np.float32)
        for sp in (1, 2):
            Y = linear_dev(h, to_dev(X, DT_BF16), N, splits=sp).cpu().numpy()
            assert np.array_equal(Y, expect)
    finally:
        sdg.spense_free(h)


def test_gather_equals_contiguous_bitwise():
    """(X, W, chosen set) and (X[:, pi], W[:, pi], tail) take the same K order: identical bits."""
    N, K, M = 96, 1024, 9
    W, s = _small(N, K, DT_FP8, 11)
    D = synth.random_dense_set(K, 256, 12)
    X = synth.make_x(M, K, DT_BF16, np.random.default_rng(13))
    pi, K_s, K_d = oracle.resolve_dense_set(K, dense_cols=D)
    sd = to_dev(s, DT_F32)
    h1 = pack_dev(to_dev(W, DT_FP8), DT_FP8, sd, dense_cols=D)
    h2 = pack_dev(to_dev(np.ascontiguousarray(W[:, pi]), DT_FP8), DT_FP8, sd, dense_fraction=K_d / K)
    try:
        assert sdg.spense_info(h1)["gather"] == 1 and sdg.spense_info(h2)["gather"] == 0
        for sp in (1, 4):
            y1 = linear_dev(h1, to_dev(X, DT_BF16), N, splits=sp)
            y2 = linear_dev(h2, to_dev(np.ascontiguousarray(X[:, pi]), DT_BF16), N, splits=sp)
            assert torch.equal(y1, y2)
    finally:
        sdg.spense_free(h1)
        sdg.spense_free(h2)


@pytest.mark.parametrize("K,K_d,M,ldx_pad", [(1000, 248, 1100, 0), (1024, 256, 1030, 3), (7168, 1792, 1040, 0)])
def test_large_batch_gather_equals_contiguous_bitwise(K, K_d, M, ldx_pad):
    """Large batches gather X'p in a pre-pass that stages whole rows in LDS
    (several rows per workgroup; K = 1000 and a leading dimension of K + 3
    take the element-wise staging): the output equals the pre-permuted
    contiguous call bit for bit."""
    N = 64
    W, s = _small(N, K, DT_FP8, 21)
    D = synth.random_dense_set(K, K_d, 22)
    X = synth.make_x(M, K, DT_BF16, np.random.default_rng(23))
    pi, K_s, _ = oracle.resolve_dense_set(K, dense_cols=D)
    sd = to_dev(s, DT_F32)
    h1 = pack_dev(to_dev(W, DT_FP8), DT_FP8, sd, dense_cols=D)
    h2 = pack_dev(to_dev(np.ascontiguousarray(W[:, pi]), DT_FP8), DT_FP8, sd, dense_fraction=K_d / K)
    try:
        Xd = to_dev(X, DT_BF16)
        if ldx_pad:
            buf = torch.zeros((M, K + ldx_pad), dtype=torch.bfloat16, device="cuda")
            buf[:, :K].copy_(Xd)
            Xd = buf[:, :K]
        y1 = linear_dev(h1, Xd, N)
        y2 = linear_dev(h2, to_dev(np.ascontiguousarray(X[:, pi]), DT_BF16), N)
        assert torch.equal(y1, y2)
    finally:
        sdg.spense_free(h1)
        sdg.spense_free(h2)


def test_power_of_two_scaling_and_determinism():
    N, K, M = 80, 768, 12
    W, s = _small(N, K, DT_FP8, 14)
    X = synth.make_x(M, K, DT_BF16, np.random.default_rng(15))
    h = pack_dev(to_dev(W, DT_FP8), DT_FP8, to_dev(s, DT_F32), dense_fraction=0.25)
    try:
        Xd = to_dev(X, DT_BF16)
        for sp in (1, 5):
            y = linear_dev(h, Xd, N, splits=sp)
            y_again = linear_dev(h, Xd, N, splits=sp)
            assert torch.equal(y, y_again)
            y4 = linear_dev(h, (Xd.float() * 4.0).to(torch.bfloat16), N, splits=sp)
            assert torch.equal(y4, y * 4.0)
    finally:
        sdg.spense_free(h)


def test_non_default_stream_and_strided_operands():
    N, K, M = 64, 512, 6
    W, s = _small(N, K, DT_FP8, 16)
    X = synth.make_x(M, K, DT_BF16, np.random.default_rng(17))
    D = synth.random_dense_set(K, 128, 18)
    Wbig = torch.zeros((N, K + 64), dtype=torch.uint8, device="cuda")
    Wbig[:, :K] = to_dev(W, DT_FP8)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        h = sdg.spense_pack(Wbig, DT_FP8, scales=to_dev(s, DT_F32), dense_cols=D, K=K, ldw=K + 64, stream=st)
        Xbig = torch.zeros((M, K + 24), dtype=torch.bfloat16, device="cuda")
        Xbig[:, :K] = to_dev(X, DT_BF16)
        Ybig = torch.full((M, N + 8), -7.0, dtype=torch.float32, device="cuda")
        sdg.spense_linear(h, Xbig, Ybig, M=M, ldx=K + 24, ldy=N + 8, stream=st)
    st.synchronize()
    try:
        ref = oracle_pack_rows(W, DT_FP8, D)
        Yref, B = oracle.linear_ref(X, DT_BF16, ref, s)
        Yb = Ybig.cpu().numpy()
        assert tol_ratio(Yb[:, :N], Yref, B) <= 1.0
        assert np.all(Yb[:, N:] == -7.0)  # padding columns untouched
    finally:
        sdg.spense_free(h)


DECODE_VARIANTS = ["4,4,0", "4,8,0", "8,4,0", "8,8,0", "4,4,1", "4,8,1", "8,4,1", "8,8,1"]


@pytest.mark.parametrize("wdtype", [DT_FP8, DT_BF16])
@pytest.mark.parametrize("dense", [("frac", 0.25), ("rand", 192)])
def test_decode_variants(wdtype, dense, monkeypatch):
    """Every decode-kernel variant (waves per workgroup, ring depth, single-shot
    or chunked activation staging) and several split counts agree with the
    oracle."""
    N, K = 200, 1536
    W, s = _small(N, K, wdtype, 21)
    X = synth.make_x(16, K, DT_BF16, np.random.default_rng(22))
    sd = to_dev(s, DT_F32) if s is not None else None
    if dense[0] == "frac":
        h = pack_dev(to_dev(W, wdtype), wdtype, sd, dense_fraction=dense[1])
        pi, K_s, _ = oracle.resolve_dense_set(K, dense_fraction=dense[1])
        D = np.sort(pi[K_s:])
    else:
        D = synth.random_dense_set(K, dense[1], 23)
        h = pack_dev(to_dev(W, wdtype), wdtype, sd, dense_cols=D)
    try:
        ref = oracle_pack_rows(W, wdtype, D)
        Xd = to_dev(X, DT_BF16)
        for v in DECODE_VARIANTS:
            monkeypatch.setenv("SPENSE_DECODE", v)
            for M in (1, 5, 16):
                Yref, B = oracle.linear_ref(X[:M], DT_BF16, ref, s)
                for sp in (0, 1, 3, 9):
                    Y = linear_dev(h, Xd[:M], N, splits=sp).cpu().numpy()
                    r = tol_ratio(Y, Yref, B)
                    assert r <= 1.0, (v, M, sp, r)
        log(f"[decode variants] wdtype={wdtype} dense={dense}: all variants within tolerance")
    finally:
        sdg.spense_free(h)


@pytest.mark.parametrize("wdtype", [DT_FP8, DT_BF16])
@pytest.mark.parametrize("dense", [("frac", 0.25), ("rand", 1280)])
def test_single_shot_staging_beyond_64kb(wdtype, dense, monkeypatch):
    """Batch sizes whose activations exceed 64 KB of LDS but fit a CU's 160 KB
    (K = 5120 in one split, M = 7..16, a grid of fewer workgroups than CUs) run the
    single-shot decode kernel when the activations are contiguous (tail dense
    set; a chosen set is gathered and keeps chunked staging): the result equals
    the chunked kernel's bit for bit (same products, same order) and the oracle
    within tolerance.  At M = 16 the padded rows do not fit and the unpadded,
    swizzled rows run; with the tail set, activations at a leading dimension
    that is not a multiple of 8 take the register (gathering) staging into the
    same swizzled rows, and equal the aligned result bit for bit."""
    N, K = 160, 5120
    W, s = _small(N, K, wdtype, 41)
    X = synth.make_x(16, K, DT_BF16, np.random.default_rng(42))
    sd = to_dev(s, DT_F32) if s is not None else None
    if dense[0] == "frac":
        h = pack_dev(to_dev(W, wdtype), wdtype, sd, dense_fraction=dense[1])
        pi, K_s, _ = oracle.resolve_dense_set(K, dense_fraction=dense[1])
        D = np.sort(pi[K_s:])
    else:
        D = synth.random_dense_set(K, dense[1], 43)
        h = pack_dev(to_dev(W, wdtype), wdtype, sd, dense_cols=D)
    try:
        ref = oracle_pack_rows(W, wdtype, D)
        Xd = to_dev(X, DT_BF16)
        Xu = torch.zeros((16, K + 1), dtype=torch.bfloat16, device="cuda")[:, :K]  # leading dimension K + 1
        Xu.copy_(Xd)
        for M in (7, 8, 12, 15, 16):
            Yref, B = oracle.linear_ref(X[:M], DT_BF16, ref, s)
            # one split: the whole K range (M x 5128 bf16 = 72-154 KB; 160 KB unpadded at M = 16) staged at once
            monkeypatch.delenv("SPENSE_DECODE", raising=False)
            Y1 = linear_dev(h, Xd[:M], N, splits=1).cpu().numpy()
            if dense[0] == "frac" and M >= 12:
                Yu = linear_dev(h, Xu[:M], N, splits=1).cpu().numpy()
                assert np.array_equal(Y1, Yu), ("unaligned", M)
            monkeypatch.setenv("SPENSE_DECODE", "8,4,1")  # chunked staging
            Y2 = linear_dev(h, Xd[:M], N, splits=1).cpu().numpy()
            assert np.array_equal(Y1, Y2), M
            r = tol_ratio(Y1, Yref, B)
            assert r <= 1.0, (M, r)
        log(f"[single-shot > 64 KB] wdtype={wdtype} dense={dense}: equal to chunked, within tolerance")
    finally:
        sdg.spense_free(h)


TILE_PRESETS = list(range(17))


@pytest.mark.parametrize("wdtype", [DT_FP8, DT_BF16])
@pytest.mark.parametrize("dense", [("frac", 0.25), ("rand", 192)])
def test_tile_presets(wdtype, dense, monkeypatch):
    """Every register-blocked configuration of the streaming kernel (row tiles
    and m-tiles per wave, ring depth, chunk size), on ragged row counts, batch
    sizes that end mid m-tile, several split counts, and a chosen dense set
    (gathered into the workspace first), agrees with the oracle."""
    N, K = 232, 1536  # 14.5 row tiles: the last row group is partial for every blocking
    W, s = _small(N, K, wdtype, 31)
    X = synth.make_x(130, K, DT_BF16, np.random.default_rng(32))
    sd = to_dev(s, DT_F32) if s is not None else None
    if dense[0] == "frac":
        h = pack_dev(to_dev(W, wdtype), wdtype, sd, dense_fraction=dense[1])
        pi, K_s, _ = oracle.resolve_dense_set(K, dense_fraction=dense[1])
        D = np.sort(pi[K_s:])
    else:
        D = synth.random_dense_set(K, dense[1], 33)
        h = pack_dev(to_dev(W, wdtype), wdtype, sd, dense_cols=D)
    try:
        ref = oracle_pack_rows(W, wdtype, D)
        Xd = to_dev(X, DT_BF16)
        for v in TILE_PRESETS:
            monkeypatch.setenv("SPENSE_TILE", str(v))
            for M in (17, 40, 64, 130):
                Yref, B = oracle.linear_ref(X[:M], DT_BF16, ref, s)
                for sp in (0, 1, 3):
                    Y = linear_dev(h, Xd[:M], N, splits=sp).cpu().numpy()
                    r = tol_ratio(Y, Yref, B)
                    assert r <= 1.0, (v, M, sp, r)
        log(f"[tile presets] wdtype={wdtype} dense={dense}: all presets within tolerance")
    finally:
        sdg.spense_free(h)


LDS_PRESETS = list(range(8))


@pytest.mark.parametrize("wdtype", [DT_FP8, DT_BF16])
@pytest.mark.parametrize("dense", [("frac", 0.25), ("rand", 192)])
def test_lds_tile_presets(wdtype, dense, monkeypatch):
    """Every configuration of the kernel that stages weight units through LDS
    for waves splitting the tokens (waves per workgroup, m-tiles per wave, row
    tiles per workgroup, unit-steps per stage), on ragged row counts, batches
    ending mid m-tile, one or several m-groups, several split counts and a
    chosen dense set, agrees with the oracle."""
    N, K = 232, 1536  # 14.5 row tiles: the last row group is partial for every configuration
    W, s = _small(N, K, wdtype, 34)
    X = synth.make_x(300, K, DT_BF16, np.random.default_rng(35))
    sd = to_dev(s, DT_F32) if s is not None else None
    if dense[0] == "frac":
        h = pack_dev(to_dev(W, wdtype), wdtype, sd, dense_fraction=dense[1])
        pi, K_s, _ = oracle.resolve_dense_set(K, dense_fraction=dense[1])
        D = np.sort(pi[K_s:])
    else:
        D = synth.random_dense_set(K, dense[1], 36)
        h = pack_dev(to_dev(W, wdtype), wdtype, sd, dense_cols=D)
    try:
        ref = oracle_pack_rows(W, wdtype, D)
        Xd = to_dev(X, DT_BF16)
        worst = 0.0
        for v in LDS_PRESETS:
            monkeypatch.setenv("SPENSE_LDS", str(v))
            for M in (17, 40, 64, 130, 300):
                Yref, B = oracle.linear_ref(X[:M], DT_BF16, ref, s)
                for sp in (0, 1, 3):
                    Y = linear_dev(h, Xd[:M], N, splits=sp).cpu().numpy()
                    r = tol_ratio(Y, Yref, B)
                    assert r <= 1.0, (v, M, sp, r)
                    worst = max(worst, r)
        log(f"[lds presets] wdtype={wdtype} dense={dense}: all configurations within tolerance (worst {worst:.2e})")
    finally:
        sdg.spense_free(h)


def test_lds_tile_equals_streaming_bitwise_on_one_split():
    """With one split both M > 16 kernels add the same products per output in
    the same unit order (sparse units, then dense units, two instructions per
    unit, fp32 accumulators), so on the same packed layer they agree bit for bit."""
    N, K, M = 160, 1024, 64
    W, s = _small(N, K, DT_FP8, 37)
    sd = to_dev(s, DT_F32)
    h = pack_dev(to_dev(W, DT_FP8), DT_FP8, sd, dense_fraction=0.25)
    try:
        Xd = to_dev(synth.make_x(M, K, DT_BF16, np.random.default_rng(38)), DT_BF16)
        import os
        os.environ["SPENSE_LDS"] = "1"
        try:
            y_lds = linear_dev(h, Xd, N, splits=1)
        finally:
            del os.environ["SPENSE_LDS"]
        os.environ["SPENSE_TILE"] = "3"  # eight waves, one row tile and four m-tiles each
        try:
            y_str = linear_dev(h, Xd, N, splits=1)
        finally:
            del os.environ["SPENSE_TILE"]
        assert torch.equal(y_lds, y_str)
    finally:
        sdg.spense_free(h)


@pytest.mark.parametrize("kernel", [("SPENSE_TILE", "0"), ("SPENSE_LDS", "4")])
def test_workgroup_order_blocks_bitwise(kernel, monkeypatch):
    """The workgroup order with several m-groups (blocks of row groups, one
    m-group at a time) only decides which workgroup computes which tile: every
    block size, including blocks that do not divide the row groups and a last
    partial block, gives the same output bit for bit, with one split and with
    several, and within tolerance of the oracle."""
    N, K = 648, 1024  # 40.5 row tiles: several row groups of either kernel, the last one partial
    W, s = _small(N, K, DT_FP8, 41)
    sd = to_dev(s, DT_F32)
    D = synth.random_dense_set(K, 256, 42)
    h = pack_dev(to_dev(W, DT_FP8), DT_FP8, sd, dense_cols=D)
    try:
        X = synth.make_x(300, K, DT_BF16, np.random.default_rng(43))
        Xd = to_dev(X, DT_BF16)
        ref = oracle_pack_rows(W, DT_FP8, D)
        monkeypatch.setenv(*kernel)
        for M in (100, 300):
            Yref, B = oracle.linear_ref(X[:M], DT_BF16, ref, s)
            for sp in (1, 3):
                ys = []
                for rb in ("1", "2", "3", "4", "5", "16"):
                    monkeypatch.setenv("SPENSE_RBLOCK", rb)
                    ys.append(linear_dev(h, Xd[:M], N, splits=sp))
                for y in ys[1:]:
                    assert torch.equal(y, ys[0]), (kernel, M, sp)
                assert tol_ratio(ys[0].cpu().numpy(), Yref, B) <= 1.0, (kernel, M, sp)
        log(f"[workgroup order] {kernel}: block sizes 1-5, 16 bitwise equal")
    finally:
        sdg.spense_free(h)
