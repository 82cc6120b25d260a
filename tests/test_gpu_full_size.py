"""GPU parity at the benchmark shapes, through the C interface, against the oracle.

Every configuration the benchmark runs is checked here at its full size and
in the launch configuration the benchmark uses (automatic plan):
  * spense_pack's canonical export bit for bit on every row (for the sets of
    the dense-fraction sweep other than 25% and the bf16 36B-class set, on 26
    spread row tiles), the oracle packing row blocks of 4096;
  * spense_linear on every output column, for every token up to M = 128 and
    64 sampled tokens at M = 2048, within 1e-3 * sum_k |x_k w_k| per element;
  * the gate/up projection in output-split form through spense_pack_rows /
    spense_export_rows / spense_linear, every row and column;
  * the GLU block at its bench shape through spense_pack_glu / spense_glu:
    the bf16 intermediate against the oracle's (the bound of the small GLU
    tests) and the block output against the oracle's down projection of the
    device's own intermediate.
SpenseGPT explainer, Technical Summary 2.A (format, input- and output-split)
and 2.B (dense set permuted into one block).
"""

from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import sparse_dense_gemm_amd as sdg
import synth
from synth import DT_BF16, DT_F32, DT_FP8

from spense_gpu_util import TOL, export, linear_dev, log, pack_dev, storage_torch_dtype, to_dev, tol_ratio

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS
BLOCK = 4096  # oracle row block
SAMPLED = {"layer32b_fp8_d0", "layer32b_fp8_d12p5", "layer32b_fp8_d50", "layer32b_fp8_d100", "layer36b_bf16"}


def _cases():
    cases = []
    for key, w in WL.items():
        if w.extra.get("glu"):
            continue
        for spec in w.layers:
            if spec.form != "input":
                continue
            cases.append((spec.layer_index, spec.wdtype, key, spec.name))
    # equal layers (same seeds, same W) next to each other so the weights are drawn once
    cases.sort(key=lambda c: (c[2].startswith("layer32b"), c[0], c[1], c[2]))
    return [(c[2], c[3]) for c in cases]


@functools.lru_cache(maxsize=1)
def _weights(N, K, wdtype, layer_index, single):
    spec = synth.LayerSpec("w", N, K, 0, wdtype, DT_F32 if wdtype == DT_F32 else DT_BF16, "tail", layer_index)
    W, s, _, _ = synth.layer_inputs(spec, 1, single_stream=single)
    return W, s


def _spread_rows(N):
    NT = (N + 15) // 16
    tiles = np.unique(np.concatenate([np.linspace(0, NT - 1, 24).astype(np.int64), [0, NT - 1]]))
    return np.concatenate([np.arange(16 * t, min(N, 16 * t + 16)) for t in tiles])


def _token_rows(M):
    if M <= 128:
        return np.arange(M)
    return np.unique(np.concatenate([np.random.default_rng(M).choice(M, 62, replace=False), [0, M - 1]]))


def _blocks(rows):
    for r0 in range(0, len(rows), BLOCK):
        yield rows[r0:r0 + BLOCK]


def _compare_pack(got, W, wdtype, pi, K_s, rows):
    """Device export (already restricted to `rows`) against the oracle, block by block."""
    pos = 0
    for blk in _blocks(rows):
        ref = oracle.pack(W[blk], wdtype, pi, K_s)
        sl = slice(pos, pos + len(blk))
        assert np.array_equal(got["mask"][sl], ref.mask), ("mask", int(blk[0]))
        assert np.array_equal(got["meta"][sl], ref.meta), ("meta", int(blk[0]))
        assert np.array_equal(got["vals"][sl].view(np.uint8), np.ascontiguousarray(ref.vals).view(np.uint8)), "vals"
        assert np.array_equal(got["dense"][sl].view(np.uint8), np.ascontiguousarray(ref.dense).view(np.uint8)), "dense"
        pos += len(blk)
    assert np.array_equal(got["pi"], pi.astype(np.int32)), "pi"


def _linear_ratio(Y, X, xdtype, W, wdtype, s, pi, K_s, rows, mrows):
    """max error / tolerance of Y[mrows][:, rows] over oracle row blocks."""
    worst = 0.0
    for blk in _blocks(rows):
        ref = oracle.pack(W[blk], wdtype, pi, K_s)
        Yref, B = oracle.linear_ref(X[mrows], xdtype, ref, None if s is None else s[blk])
        worst = max(worst, tol_ratio(Y[np.ix_(mrows, blk)], Yref, B))
    return worst


@pytest.mark.parametrize("key,lname", _cases())
def test_workload_full_size(key, lname):
    w = WL[key]
    spec = next(s for s in w.layers if s.name == lname)
    Mmax = max(w.Ms)
    full = key not in SAMPLED
    log(f"[full size] {key}/{lname} N={spec.N} K={spec.K} K_d={spec.K_d} wdtype={spec.wdtype} Ms={w.Ms} "
        f"rows={'all' if full else 'spread'}")
    W, s = _weights(spec.N, spec.K, spec.wdtype, spec.layer_index, w.single_stream)
    if w.single_stream:
        _, _, X, D = synth.layer_inputs(spec, Mmax, single_stream=True)
    else:
        _, _, X, D = synth.layer_inputs(synth.LayerSpec(spec.name, 1, spec.K, spec.K_d, spec.wdtype, spec.xdtype,
                                                        spec.dense, spec.layer_index), Mmax)
    rows = np.arange(spec.N) if full else _spread_rows(spec.N)
    pi, K_s, _ = oracle.resolve_dense_set(spec.K, dense_cols=D)
    h = pack_dev(to_dev(W, spec.wdtype), spec.wdtype, to_dev(s, DT_F32) if s is not None else None, dense_cols=D)
    try:
        got = export(h, spec.wdtype, None if full else rows)
        _compare_pack(got, W, spec.wdtype, pi, K_s, rows)
        log(f"  pack bit-exact on {len(rows)} of {spec.N} rows")
        del got
        Xd = to_dev(X, spec.xdtype)
        for M in w.Ms:
            Y = linear_dev(h, Xd[:M], spec.N).cpu().numpy()
            mrows = _token_rows(M)
            r = _linear_ratio(Y, X, spec.xdtype, W, spec.wdtype, s, pi, K_s, rows, mrows)
            log(f"  M={M}: {len(mrows)} tokens x {len(rows)} columns, max err / (1e-3 * sum|xw|) = {r:.3e}")
            assert r <= 1.0
    finally:
        sdg.spense_free(h)


def test_output_split_bench_shape():
    """gate/up 25600 x 5120 e4m3 in output-split form, the last 6400 rows dense
    (the benchmark's gateup_fp8_rows): export of every row, every output column."""
    spec = WL["gateup_fp8_rows"].layers[0]
    W, s, X, _ = synth.layer_inputs(spec, 16)
    N, K = spec.N, spec.K
    dense_rows = np.arange(N - spec.N_d, N, dtype=np.int32)
    h = sdg.spense_pack_rows(to_dev(W, DT_FP8), DT_FP8, scales=to_dev(s, DT_F32), dense_rows=dense_rows)
    try:
        info = sdg.spense_info(h)
        assert (info["N_s"], info["N_d"]) == (N - spec.N_d, spec.N_d)
        N_s = info["N_s"]
        sd = storage_torch_dtype(DT_FP8)
        vals = torch.empty((N_s, K // 2), dtype=sd, device="cuda")
        meta = torch.empty((N_s, (K // 4 + 7) // 8), dtype=torch.int32, device="cuda")
        mask = torch.empty((N_s, K), dtype=torch.uint8, device="cuda")
        dense = torch.empty((spec.N_d, K), dtype=sd, device="cuda")
        rho = sdg.spense_export_rows(h, vals, meta, mask, dense)
        rho_ref, N_s_ref, _ = oracle.resolve_dense_rows(N, K, dense_rows=dense_rows)
        assert np.array_equal(rho, rho_ref.astype(np.int32)) and N_s_ref == N_s
        vals, meta, mask = vals.cpu().numpy(), meta.cpu().numpy().view(np.uint32), mask.cpu().numpy()
        ident = np.arange(K)
        for r0 in range(0, N_s, BLOCK):
            blk = rho_ref[r0:min(N_s, r0 + BLOCK)]
            ref = oracle.pack(W[blk], DT_FP8, ident, K)
            sl = slice(r0, r0 + len(blk))
            assert np.array_equal(mask[sl], ref.mask) and np.array_equal(meta[sl], ref.meta), r0
            assert np.array_equal(vals[sl], ref.vals), r0
        assert np.array_equal(dense.cpu().numpy(), W[rho_ref[N_s:]])
        log(f"[full size] output-split gate/up: export bit-exact on all {N} rows")
        Xd = to_dev(X, DT_BF16)
        P = oracle.pack_rows(W, DT_FP8, rho_ref, N_s)
        for M in WL["gateup_fp8_rows"].Ms:
            Y = linear_dev(h, Xd[:M], N).cpu().numpy()
            Yref, B = oracle.linear_rows_ref(X[:M], DT_BF16, P, s)
            r = tol_ratio(Y, Yref, B)
            log(f"  M={M}: every column, max err / tolerance = {r:.3e}")
            assert r <= 1.0
    finally:
        sdg.spense_free(h)


def _a_tolerance(r):
    """bf16 rounding of silu(G) * U (2^-9 relative, doubled to cover the fp32
    SiLU) plus the layer tolerance of G and U carried through (|silu'| < 1.1)."""
    G, U, A = r["G"], r["U"], r["A"]
    eG, eU = TOL * r["B_G"], TOL * r["B_U"]
    return 2.0 ** -8 * np.abs(A) + 1.1 * eG * (np.abs(U) + eU) + np.abs(oracle.silu(G)) * eU


def test_glu_bench_shape():
    """The GLU block at the benchmark's shape (glu32b_fp8: H 5120, I 25600,
    6400 chosen dense intermediate indices), M in {1, 4, 16}."""
    wl = WL["glu32b_fp8"]
    gu, dn = wl.layers
    H, I = dn.N, dn.K
    Wgu, sgu, X, _ = synth.layer_inputs(gu, max(wl.Ms))
    Wd, sd, _, D = synth.layer_inputs(dn, max(wl.Ms))
    h = sdg.spense_pack_glu(to_dev(Wgu, DT_FP8), to_dev(Wd, DT_FP8), DT_FP8, H=H, I=I, s_gu=to_dev(sgu, DT_F32),
                            s_down=to_dev(sd, DT_F32), dense_idx=D)
    try:
        Xd = to_dev(X, DT_BF16)
        pi, K_s, _ = oracle.resolve_dense_set(I, dense_cols=D)
        Pd = oracle.pack(Wd, DT_FP8, pi, K_s)
        for M in wl.Ms:
            A = torch.empty((M, I), dtype=torch.bfloat16, device="cuda")
            Y = torch.empty((M, H), dtype=torch.float32, device="cuda")
            sdg.spense_glu(h, Xd[:M], A, Y)
            torch.cuda.synchronize()
            r = oracle.glu_block_ref(X[:M], DT_BF16, Wgu[:I], Wgu[I:], Wd, DT_FP8, D, sgu[:I], sgu[I:], sd)
            rho = r["rho"]
            a_dev = A.float().cpu().numpy().astype(np.float64)  # rho order
            err_a = np.abs(a_dev - r["A"][:, rho])
            tol_a = _a_tolerance(r)[:, rho]
            assert np.all(err_a <= tol_a + 1e-30), (M, float(np.max(err_a - tol_a)))
            a_nat = np.zeros_like(a_dev)
            a_nat[:, rho] = a_dev
            Yref, B = oracle.down_ref(a_nat, Pd, sd)
            ry = tol_ratio(Y.cpu().numpy(), Yref, B)
            log(f"[full size] GLU block M={M}: intermediate {float(np.max(err_a / (tol_a + 1e-30))):.2e}, "
                f"output {ry:.2e} of tolerance")
            assert ry <= 1.0
    finally:
        sdg.spense_free(h)


@pytest.mark.parametrize("a8", [False, True], ids=["w8a16", "w8a8"])
def test_down_projection_between_benchmark_batches(a8):
    """The 36B-class down projection (5120 x 27648, 6912 chosen dense
    columns) at batch sizes between the benchmark's, where the launch planner
    moves to larger tiles with split-K (M > 128) or to two-row-tile tiles with
    splits (M = 96): automatic plan, a spread sample of row tiles for a sample
    of tokens, against the oracle (W8A8: the exact W8A8 result of the oracle's
    own per-token codes)."""
    spec = next(x for x in WL["layer36b_fp8"].layers if x.name == "down")
    Ms = (96, 192, 256, 384, 512)
    W, s, X, D = synth.layer_inputs(spec, max(Ms))
    rows = _spread_rows(spec.N)
    pi, K_s, _ = oracle.resolve_dense_set(spec.K, dense_cols=D)
    ref = oracle.pack(W[rows], DT_FP8, pi, K_s)
    h = pack_dev(to_dev(W, DT_FP8), DT_FP8, to_dev(s, DT_F32), dense_cols=D)
    try:
        Xd = to_dev(X, DT_BF16)
        for M in Ms:
            sel = np.unique(np.concatenate([np.random.default_rng(7 + M).choice(M, 30, replace=False), [0, M - 1]]))
            Y = torch.empty((M, spec.N), dtype=torch.float32, device="cuda")
            if a8:
                sdg.spense_linear_w8a8(h, Xd[:M], Y)
                q, sx = oracle.quantize_tokens_ref(X[sel], DT_BF16)
                Yref, B = oracle.linear_w8a8_ref(q, sx, ref, s[rows])
            else:
                sdg.spense_linear(h, Xd[:M], Y)
                Yref, B = oracle.linear_ref(X[sel], DT_BF16, ref, s[rows])
            torch.cuda.synchronize()
            r = tol_ratio(Y.cpu().numpy()[np.ix_(sel, rows)], Yref, B)
            log(f"[down between batches] {'w8a8' if a8 else 'w8a16'} M={M}: ratio {r:.3e} "
                f"on {sel.size} tokens x {rows.size} rows")
            assert r <= 1.0
    finally:
        sdg.spense_free(h)
