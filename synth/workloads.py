"""The five synthetic Spense workloads (shapes, dtypes, dense sets, batch sizes).

Every layer is Y[M,N] = X[M,K] . W[N,K]^T with K split into a 2:4 region and a
dense region of K_d columns.  Seeds: a single-layer workload uses W seed 0,
X seed 1 and dense-set seed 2; layer j of a multi-layer set uses seeds 3j,
3j+1 and 3j+2.  The small fp32 layer draws W and then X from one seed-0
stream.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

from .gen import DT_BF16, DT_F32, DT_FP8, make_weight, make_x, random_dense_set, tail_dense_set


@dataclass(frozen=True)
class LayerSpec:
    name: str
    N: int
    K: int
    K_d: int
    wdtype: int
    xdtype: int
    dense: str  # "tail" or "random"
    layer_index: int = 0
    form: str = "input"  # "input": dense columns (K_d of them); "output": dense rows (N_d of them), K_d = 0
    N_d: int = 0


@dataclass
class Workload:
    key: str
    title: str
    layers: List[LayerSpec]
    Ms: Tuple[int, ...]
    single_stream: bool = False
    extra: dict = field(default_factory=dict)


def _set(prefix, shapes, wdt, xdt, frac_or_kd, dense):
    out = []
    for j, (nm, N, K) in enumerate(shapes):
        if isinstance(frac_or_kd, dict):
            K_d = frac_or_kd[nm]
        else:
            K_d = int(round(frac_or_kd * K))
        out.append(LayerSpec(f"{prefix}{nm}", N, K, K_d, wdt, xdt, dense, j))
    return out


_SHAPES_32B = [("qkv", 10240, 5120), ("o", 5120, 8192), ("gateup", 51200, 5120), ("down", 5120, 25600)]
_SHAPES_36B = [("qkv", 12288, 5120), ("o", 5120, 10240), ("gateup", 55296, 5120), ("down", 5120, 27648)]


def _build():
    w = {}
    w["fp32_small"] = Workload(
        "fp32_small", "fp32 layer W[256,512], 128-column dense tail, M=1",
        [LayerSpec("small", 256, 512, 128, DT_F32, DT_F32, "tail")], (1,), single_stream=True)
    w["gateup_fp8"] = Workload(
        "gateup_fp8", "32B-class FFN gate/up W[25600,5120] e4m3, dense tail 1280, M in {1,4,16}",
        [LayerSpec("gateup", 25600, 5120, 1280, DT_FP8, DT_BF16, "tail")], (1, 4, 16))
    w["gateup_fp8_rows"] = Workload(
        "gateup_fp8_rows", "32B-class FFN gate/up W[25600,5120] e4m3, output-split with the last 6400 rows dense, "
        "M in {1,4,16}",
        [LayerSpec("gateup_rows", 25600, 5120, 0, DT_FP8, DT_BF16, "tail", form="output", N_d=6400)], (1, 4, 16))
    w["glu32b_fp8"] = Workload(
        "glu32b_fp8", "32B-class GLU MLP block H=5120, I=25600, e4m3: gate/up output-split and down input-split over "
        "6400 chosen dense intermediate indices, M in {1,4,16}",
        [LayerSpec("gate_up", 51200, 5120, 0, DT_FP8, DT_BF16, "tail", 0),
         LayerSpec("down", 5120, 25600, 6400, DT_FP8, DT_BF16, "random", 1)], (1, 4, 16), extra={"glu": True})
    w["down_fp8"] = Workload(
        "down_fp8", "32B-class FFN down W[5120,25600] e4m3, 6400 random dense columns, M in {1,8,32,64}",
        [LayerSpec("down", 5120, 25600, 6400, DT_FP8, DT_BF16, "random")], (1, 8, 32, 64))
    for frac, tag in ((0.0, "0"), (0.125, "12p5"), (0.25, "25"), (0.5, "50"), (1.0, "100")):
        w[f"layer32b_fp8_d{tag}"] = Workload(
            f"layer32b_fp8_d{tag}", f"32B-class decoder linear set, e4m3, dense tail fraction {frac}, M=32",
            _set("", _SHAPES_32B, DT_FP8, DT_BF16, frac, "tail"), (32,), extra={"fraction": frac})
    kd36 = {"qkv": 1280, "o": 2560, "gateup": 1280, "down": 6912}
    w["layer36b_fp8"] = Workload(
        "layer36b_fp8", "36B-class decoder linear set, e4m3, 25% random dense columns, M in {128,2048}",
        _set("", _SHAPES_36B, DT_FP8, DT_BF16, kd36, "random"), (128, 2048))
    w["layer36b_bf16"] = Workload(
        "layer36b_bf16", "36B-class decoder linear set, bf16, 25% random dense columns, M in {128,2048}",
        _set("", _SHAPES_36B, DT_BF16, DT_BF16, kd36, "random"), (128, 2048))
    return w


WORKLOADS = _build()


def layer_inputs(spec: LayerSpec, M: int, single_stream: bool = False, rows: Optional[int] = None):
    """Draw (W bits, scales, X bits, dense set) for one layer at batch M.

    ``rows`` limits the draw to the first ``rows`` output channels (the stream
    is row-major, so those rows are identical to the full draw's).
    """
    N = spec.N if rows is None else min(rows, spec.N)
    j = spec.layer_index
    if single_stream:
        rng = np.random.default_rng(0)
        W, s = make_weight(spec.N, spec.K, spec.wdtype, rng)
        X = make_x(M, spec.K, spec.xdtype, rng)
        W = W[:N]
        s = None if s is None else s[:N]
    else:
        W, s = make_weight(N, spec.K, spec.wdtype, np.random.default_rng(3 * j))
        X = make_x(M, spec.K, spec.xdtype, np.random.default_rng(3 * j + 1))
    if spec.dense == "tail":
        D = tail_dense_set(spec.K, spec.K_d)
    else:
        D = random_dense_set(spec.K, spec.K_d, 3 * j + 2)
    return W, s, X, D
