"""GPU parity of the GLU block (spense_pack_glu / spense_glu) against the oracle.

SpenseGPT explainer, Technical Summary 2.A / 2.B: gate and up output-split,
down input-split, one dense set of intermediate indices moved into a
contiguous block at pack time.  The intermediate silu(gate) * up is checked
against the oracle's (it is rounded to bf16 on the device), and the block
output against the oracle's down projection of the device's own
intermediate, with the layer tolerance.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sparse_dense_gemm_amd as sdg
import synth
from synth import DT_BF16, DT_F32, DT_FP8

from spense_gpu_util import TOL, log, to_dev, tol_ratio

pytestmark = pytest.mark.gpu

CASES = [
    # (H, I, wdtype, dense intermediate set)
    (256, 512, DT_FP8, ("frac", 0.25)),
    (256, 512, DT_BF16, ("rand", 100)),
    (132, 388, DT_FP8, ("rand", 64)),    # ragged H and I
    (128, 256, DT_FP8, ("frac", 0.0)),   # no dense index
    (128, 256, DT_BF16, ("frac", 1.0)),  # every index dense
]


def _inputs(H, I, wdt, seed):
    rng = np.random.default_rng(seed)
    Wgu, sgu = synth.make_weight(2 * I, H, wdt, rng)
    Wd, sd = synth.make_weight(H, I, wdt, rng)
    X = synth.make_x(130, H, DT_BF16, rng)
    return Wgu, sgu, Wd, sd, X


def _dense(I, spec, seed):
    if spec[0] == "frac":
        I_d = int(np.floor(spec[1] * I + 0.5))
        return np.arange(I - I_d, I), dict(dense_fraction=spec[1])
    D = synth.random_dense_set(I, spec[1], seed)
    return D, dict(dense_idx=D)


def _a_tolerance(r):
    """Per element bound for the bf16 intermediate: bf16 rounding of the
    product (2^-9 relative, doubled to cover the fp32 SiLU), plus the layer
    tolerance on G and U carried through silu(G) * U (|silu'| < 1.1)."""
    G, U, A = r["G"], r["U"], r["A"]
    eG, eU = TOL * r["B_G"], TOL * r["B_U"]
    return 2.0 ** -8 * np.abs(A) + 1.1 * eG * (np.abs(U) + eU) + np.abs(oracle.silu(G)) * eU


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"H{c[0]}I{c[1]}w{c[2]}{c[3][0]}{c[3][1]}")
def test_glu_block(case):
    H, I, wdt, spec = case
    Wgu, sgu, Wd, sd, X = _inputs(H, I, wdt, 81)
    D, kw = _dense(I, spec, 82)
    to = (lambda a: to_dev(a, DT_F32)) if sgu is not None else (lambda a: None)
    h = sdg.spense_pack_glu(to_dev(Wgu, wdt), to_dev(Wd, wdt), wdt, H=H, I=I,
                            s_gu=to(sgu) if sgu is not None else None, s_down=to(sd) if sd is not None else None, **kw)
    try:
        info = sdg.spense_info(h)
        assert info["split"] == 2 and info["N_d"] == len(D) and info["N_s"] == I - len(D)
        Xd = to_dev(X, DT_BF16)
        worst_a = worst_y = 0.0
        for M in (1, 5, 16, 17, 64, 130):
            A = torch.empty((M, I), dtype=torch.bfloat16, device="cuda")
            Y = torch.empty((M, H), dtype=torch.float32, device="cuda")
            sdg.spense_glu(h, Xd[:M], A, Y)
            torch.cuda.synchronize()
            r = oracle.glu_block_ref(X[:M], DT_BF16, Wgu[:I], Wgu[I:], Wd, wdt, D,
                                     None if sgu is None else sgu[:I], None if sgu is None else sgu[I:], sd)
            rho = r["rho"]
            a_dev = A.float().cpu().numpy().astype(np.float64)        # rho order
            tol_a = _a_tolerance(r)[:, rho]
            err_a = np.abs(a_dev - r["A"][:, rho])
            assert np.all(err_a <= tol_a + 1e-30), (M, float(np.max(err_a - tol_a)))
            worst_a = max(worst_a, float(np.max(err_a / (tol_a + 1e-30))))
            # down projection of the device's own intermediate
            a_nat = np.zeros_like(a_dev)
            a_nat[:, rho] = a_dev
            pi, K_s, _ = oracle.resolve_dense_set(I, dense_cols=D)
            Yref, B = oracle.down_ref(a_nat, oracle.pack(Wd, wdt, pi, K_s), sd)
            ry = tol_ratio(Y.cpu().numpy(), Yref, B)
            assert ry <= 1.0, (M, ry)
            worst_y = max(worst_y, ry)
        log(f"[glu] H={H} I={I} wdtype={wdt} {spec}: intermediate {worst_a:.2e}, output {worst_y:.2e} of tolerance")
    finally:
        sdg.spense_free(h)


def test_glu_matches_separate_layers():
    """The block equals its parts run one by one: the gate and up projections
    as output-split layers (fp32 out), silu * up rounded to bf16 on the host
    side of the comparison, in rho order, then the down projection as an
    input-split layer over the permuted intermediate with its dense tail."""
    H, I, wdt = 256, 640, DT_FP8
    Wgu, sgu, Wd, sd, X = _inputs(H, I, wdt, 83)
    D = synth.random_dense_set(I, 160, 84)
    M = 16
    h = sdg.spense_pack_glu(to_dev(Wgu, wdt), to_dev(Wd, wdt), wdt, H=H, I=I, s_gu=to_dev(sgu, DT_F32),
                            s_down=to_dev(sd, DT_F32), dense_idx=D)
    hg = sdg.spense_pack_rows(to_dev(Wgu[:I], wdt), wdt, scales=to_dev(sgu[:I], DT_F32), dense_rows=D)
    hu = sdg.spense_pack_rows(to_dev(Wgu[I:], wdt), wdt, scales=to_dev(sgu[I:], DT_F32), dense_rows=D)
    try:
        Xd = to_dev(X[:M], DT_BF16)
        A = torch.empty((M, I), dtype=torch.bfloat16, device="cuda")
        Y = torch.empty((M, H), dtype=torch.float32, device="cuda")
        sdg.spense_glu(h, Xd, A, Y)
        G = torch.empty((M, I), dtype=torch.float32, device="cuda")
        U = torch.empty((M, I), dtype=torch.float32, device="cuda")
        sdg.spense_linear(hg, Xd, G)
        sdg.spense_linear(hu, Xd, U)
        torch.cuda.synchronize()
        rho = oracle.resolve_dense_rows(I, H, dense_rows=D)[0]
        a_sep = (G * torch.sigmoid(G) * U)[:, torch.as_tensor(rho, device="cuda")]
        # same products and sums, different order of the SiLU arithmetic: within a bf16 ulp
        diff = (A.float() - a_sep).abs()
        assert torch.all(diff <= 2.0 ** -7 * a_sep.abs() + 1e-30)
        log("[glu] block intermediate matches the separate output-split layers")
    finally:
        for hh in (h, hg, hu):
            sdg.spense_free(hh)
