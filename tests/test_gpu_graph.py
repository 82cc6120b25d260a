"""spense_linear / spense_linear_w8a8 / spense_glu captured in a HIP graph (through torch's
graph capture on a side stream) and replayed: every replay equals the eager
call bit for bit.  Each configuration is called once eagerly first, so its
workspaces exist before capture (a call that grows them synchronises the
stream and allocates, which a capture cannot hold); between replays the
program runs eager calls of its own.  The split-K hand-off counters are reset
by the kernels themselves, so no memory-set node enters the graph."""

import numpy as np
import pytest
import torch

import sparse_dense_gemm_amd as sdg
import synth
from synth import DT_BF16, DT_F32, DT_FP8

from spense_gpu_util import log, pack_dev, to_dev

pytestmark = pytest.mark.gpu

N, K = 320, 2048


def _layer(form):
    W, s = synth.make_weight(N, K, DT_FP8, np.random.default_rng(51))
    Wd, sd = to_dev(W, DT_FP8), to_dev(s, DT_F32)
    if form == "tail":
        return pack_dev(Wd, DT_FP8, sd, dense_fraction=0.25)
    if form == "chosen":
        return pack_dev(Wd, DT_FP8, sd, dense_cols=synth.random_dense_set(K, 512, 52))
    return sdg.spense_pack_rows(Wd, DT_FP8, scales=sd, dense_rows=np.arange(N - 64, N, dtype=np.int32))


# (layer form, batch size, forced split count or 0, W8A8)
CASES = [
    ("tail", 4, 3, False),     # single-shot decode kernel, split-K hand-off between workgroups
    ("chosen", 12, 0, False),  # chosen set gathered while staging (single-shot decode kernel), 12 splits
    ("chosen", 40, 0, False),  # gather pre-pass, register-blocked streaming kernel, two m-groups
    ("rows", 1, 0, False),     # both row classes of an output-split layer in one launch
    ("tail", 40, 0, True),     # W8A8: quantisation pass, then the e4m3 product
]


@pytest.mark.parametrize("form,M,splits,a8", CASES)
def test_graph_replays_equal_eager(form, M, splits, a8):
    h = _layer(form)
    try:
        X = to_dev(synth.make_x(M, K, DT_BF16, np.random.default_rng(53)), DT_BF16)
        Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        Y_eager = torch.empty_like(Y)

        def call(out, stream=None):
            if a8:
                sdg.spense_linear_w8a8(h, X, out, splits=splits, stream=stream)
            else:
                sdg.spense_linear_splits(h, X, out, splits, stream=stream)

        call(Y_eager)
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(Y)  # sizes the workspaces on the capture stream's handle state
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            call(Y)
        torch.cuda.synchronize()
        other = torch.empty_like(Y)
        for rep in range(3):
            Y.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(Y, Y_eager), (form, M, splits, a8, rep)
            call(other)  # eager work between replays
            torch.cuda.synchronize()
            assert torch.equal(other, Y_eager), (form, M, splits, a8, rep)
        log(f"[graph] {form} M={M} splits={splits} a8={a8}: 3 replays equal eager")
    finally:
        sdg.spense_free(h)


@pytest.mark.parametrize("M", [4, 40])
def test_graph_replays_of_the_glu_block_equal_eager(M):
    H, I = 256, 512
    Wgu, sgu = synth.make_weight(2 * I, H, DT_FP8, np.random.default_rng(61))
    Wdn, sdn = synth.make_weight(H, I, DT_FP8, np.random.default_rng(62))
    h = sdg.spense_pack_glu(to_dev(Wgu, DT_FP8), to_dev(Wdn, DT_FP8), DT_FP8, H=H, I=I, s_gu=to_dev(sgu, DT_F32),
                            s_down=to_dev(sdn, DT_F32), dense_idx=synth.random_dense_set(I, 128, 63))
    try:
        X = to_dev(synth.make_x(M, H, DT_BF16, np.random.default_rng(64)), DT_BF16)
        A, A_eager = (torch.empty((M, I), dtype=torch.bfloat16, device="cuda") for _ in range(2))
        Y, Y_eager = (torch.empty((M, H), dtype=torch.float32, device="cuda") for _ in range(2))
        sdg.spense_glu(h, X, A_eager, Y_eager)
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            sdg.spense_glu(h, X, A, Y)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            sdg.spense_glu(h, X, A, Y)
        torch.cuda.synchronize()
        A2, Y2 = torch.empty_like(A), torch.empty_like(Y)
        for rep in range(3):
            A.fill_(float("nan"))
            Y.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(A, A_eager) and torch.equal(Y, Y_eager), (M, rep)
            sdg.spense_glu(h, X, A2, Y2)  # eager work between replays
            torch.cuda.synchronize()
            assert torch.equal(Y2, Y_eager), (M, rep)
        log(f"[graph] GLU block M={M}: 3 replays equal eager")
    finally:
        sdg.spense_free(h)


@pytest.mark.parametrize("form,a8", [("chosen", False), ("rows", False), ("tail", True)])
def test_capture_at_a_smaller_batch_after_one_larger_call(form, a8):
    """One eager call at M = 128 sizes the workspaces for every smaller batch
    size, so a capture at M = 1 (a split-K decode launch, which the M = 128
    call does not use) allocates nothing; its replays equal eager calls."""
    h = _layer(form)
    try:
        Xbig = to_dev(synth.make_x(128, K, DT_BF16, np.random.default_rng(55)), DT_BF16)
        Ybig = torch.empty((128, N), dtype=torch.float32, device="cuda")

        def call(X, out, stream=None):
            if a8:
                sdg.spense_linear_w8a8(h, X, out, stream=stream)
            else:
                sdg.spense_linear(h, X, out, stream=stream)

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(Xbig, Ybig)  # the only call before the capture
        torch.cuda.synchronize()
        X1 = Xbig[:1]
        Y1 = torch.empty((1, N), dtype=torch.float32, device="cuda")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            call(X1, Y1)
        torch.cuda.synchronize()
        Y_eager = torch.empty_like(Y1)
        call(X1, Y_eager)
        torch.cuda.synchronize()
        for rep in range(3):
            Y1.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(Y1, Y_eager), (form, a8, rep)
            call(Xbig, Ybig)  # eager work at the larger batch between replays
            torch.cuda.synchronize()
        log(f"[graph] {form} a8={a8}: capture at M=1 after one call at M=128, 3 replays equal eager")
    finally:
        sdg.spense_free(h)
