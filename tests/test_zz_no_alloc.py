"""spense_linear_noalloc (workspaces in the library's fixed device scratch,
no allocation) against spense_linear (the handle's workspaces): bitwise
equal, and both within the layer tolerance of the oracle, on two calls in a
row with the second at a smaller batch; a call that needs more than the
scratch holds is refused with SPENSE_ESCRATCH before any launch."""

import numpy as np
import pytest
import torch

import oracle
import sparse_dense_gemm_amd as sdg
import synth
from synth import DT_BF16, DT_F32, DT_FP8

from spense_gpu_util import log, to_dev

pytestmark = pytest.mark.gpu

N, K = 320, 2048


def _case(form, wdt):
    W, s = synth.make_weight(N, K, wdt, np.random.default_rng(71))
    Wd = to_dev(W, wdt)
    sd = to_dev(s, DT_F32) if s is not None else None
    if form == "rows":
        rows = np.arange(N - 64, N, dtype=np.int32)
        h = sdg.spense_pack_rows(Wd, wdt, scales=sd, dense_rows=rows)
        rho, N_s, _ = oracle.resolve_dense_rows(N, K, dense_rows=rows)
        P = oracle.pack_rows(W, wdt, rho, N_s)
        return h, lambda X: oracle.linear_rows_ref(X, DT_BF16 if wdt != DT_F32 else DT_F32, P, s)
    D = synth.tail_dense_set(K, 512) if form == "tail" else synth.random_dense_set(K, 512, 72)
    h = sdg.spense_pack(Wd, wdt, scales=sd, dense_cols=D)
    pi, K_s, _ = oracle.resolve_dense_set(K, dense_cols=D)
    P = oracle.pack(W, wdt, pi, K_s)
    return h, lambda X: oracle.linear_ref(X, DT_BF16 if wdt != DT_F32 else DT_F32, P, s)


CASES = [("tail", DT_FP8, 40, 4), ("chosen", DT_FP8, 40, 4), ("chosen", DT_FP8, 16, 1), ("rows", DT_FP8, 24, 3),
         ("chosen", DT_BF16, 130, 16), ("tail", DT_F32, 5, 2)]


@pytest.mark.parametrize("form,wdt,M1,M2", CASES)
def test_noalloc_equals_linear_on_two_calls(form, wdt, M1, M2):
    print(f"[no-alloc] {form} wdtype={wdt} M={M1} then M={M2}", flush=True)
    h, ref = _case(form, wdt)
    try:
        xdt = DT_F32 if wdt == DT_F32 else DT_BF16
        X = synth.make_x(M1, K, xdt, np.random.default_rng(73))
        Xd = to_dev(X, xdt)
        for M in (M1, M2):  # the second call is smaller
            Y_ref = torch.empty((M, N), dtype=torch.float32, device="cuda")
            Y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
            sdg.spense_linear(h, Xd[:M], Y_ref)
            sdg.spense_linear_noalloc(h, Xd[:M], Y)
            torch.cuda.synchronize()
            assert torch.equal(Y, Y_ref), (form, wdt, M)
            Yo, B = ref(X[:M])
            err = np.abs(Y.cpu().numpy().astype(np.float64) - Yo)
            assert np.all(err <= 1e-3 * B), (form, wdt, M, float(np.max(err / (1e-3 * B))))
        log(f"[no-alloc] {form} wdtype={wdt} M={M1},{M2}: equal to spense_linear, within tolerance")
    finally:
        sdg.spense_free(h)


def test_noalloc_refuses_beyond_the_scratch():
    """A chosen dense set at M = 8192 gathers 8192 x 2048 bf16 activations
    (32 MiB), more than the scratch holds after its counters."""
    print("[no-alloc] refusal beyond the scratch", flush=True)
    h, _ = _case("chosen", DT_FP8)
    try:
        M = 8192
        Xd = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
        Y = torch.zeros((M, N), dtype=torch.float32, device="cuda")
        with pytest.raises(sdg.SpenseError) as e:
            sdg.spense_linear_noalloc(h, Xd, Y)
        assert e.value.status == sdg.SPENSE_ESCRATCH
        torch.cuda.synchronize()
        assert not torch.any(Y != 0)  # nothing was launched
        # the handle and the scratch still work afterwards
        sdg.spense_linear_noalloc(h, Xd[:4], Y[:4])
        torch.cuda.synchronize()
    finally:
        sdg.spense_free(h)
