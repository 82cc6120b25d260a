"""Pins of the CPU oracle against things other than itself.

Each test fixes the oracle to an outside fact: a hand-worked example, a
library routine (torch's e4m3/bf16 casts, torch's float64 GEMM), an
independent characterisation (pairwise dominance for the 2:4 choice), exact
integer brute force, or an invariant the pages state (2:4 groups hold at most
two nonzeros; permuting indices into the dense block leaves the output
unchanged).
"""

import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import DT_BF16, DT_F32, DT_FP8
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# independent helpers (not the oracle's code paths)
# --------------------------------------------------------------------------
def dominance_pair(keys):
    """The unique kept pair by pairwise dominance: P is valid iff every i in P
    beats every j outside P (larger key, or equal key and lower position)."""
    valid = []
    for P in itertools.combinations(range(4), 2):
        ok = True
        for i in P:
            for j in range(4):
                if j in P:
                    continue
                if not (keys[i] > keys[j] or (keys[i] == keys[j] and i < j)):
                    ok = False
        if ok:
            valid.append(P)
    assert len(valid) == 1, (keys, valid)
    return valid[0]


def prune_python(Wvals, keys, pi, K_s):
    """Pruned weight values in natural order, by plain loops."""
    N = len(Wvals)
    out = [[float(v) for v in row] for row in Wvals]
    for n in range(N):
        for g in range(K_s // 4):
            cols = [int(pi[4 * g + t]) for t in range(4)]
            kk = [int(keys[n][c]) for c in cols]
            keep = sorted(range(4), key=lambda t: (-kk[t], t))[:2]
            for t in range(4):
                if t not in keep:
                    out[n][cols[t]] = 0.0
    return out


def torch_e4m3_values():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


# --------------------------------------------------------------------------
# element encodings
# --------------------------------------------------------------------------
def test_e4m3_decode_matches_torch_all_codes():
    ref = torch_e4m3_values()
    got = oracle.decode_values(np.arange(256, dtype=np.uint8), DT_FP8)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))
    # closed forms: largest finite, smallest subnormal, smallest normal, one
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x38] == 1.0
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.decode_values(bits, DT_BF16)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_synth_e4m3_encoder_matches_torch_cast():
    rng = np.random.default_rng(5)
    vals = np.concatenate([
        rng.normal(0, 50, 20000), rng.normal(0, 0.01, 20000), rng.uniform(-448, 448, 20000),
        torch_e4m3_values()[np.isfinite(torch_e4m3_values())],
    ])
    # exact midpoints between neighbouring codes exercise ties-to-even
    fin = np.sort(np.unique(np.abs(torch_e4m3_values()[np.isfinite(torch_e4m3_values())])))
    mids = (fin[1:] + fin[:-1]) / 2
    vals = np.concatenate([vals, mids, -mids, [0.0, -0.0, 448.0, -448.0]])
    vals = np.clip(vals, -448, 448)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = synth.e4m3_encode(vals)
    assert np.array_equal(ref, got)
    # saturation: beyond the largest finite value the encoder clamps to 448
    assert synth.e4m3_encode(np.array([1e6, -500.0])).tolist() == [0x7E, 0xFE]


def test_synth_bf16_encoder_matches_torch_cast():
    rng = np.random.default_rng(6)
    v = np.concatenate([rng.normal(0, 1, 50000), rng.normal(0, 1e-30, 1000), [0.0, -0.0, 1.0, 3.0e38]])
    f32 = v.astype(np.float32)
    ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ref, synth.bf16_encode(v))


# --------------------------------------------------------------------------
# a1: dense-set resolution
# --------------------------------------------------------------------------
def test_dense_set_tail_and_rounding():
    pi, K_s, K_d = oracle.resolve_dense_set(5120, dense_fraction=0.25)
    assert (K_s, K_d) == (3840, 1280)
    assert np.array_equal(pi, np.arange(5120))
    for K, p, kd in ((100, 0.125, 13), (100, 0.12, 12), (8, 0.5, 4), (12, 1 / 3, 4), (16, 0.0, 0), (16, 1.0, 16)):
        if (K - kd) % 4:
            with pytest.raises(oracle.DenseSetError):
                oracle.resolve_dense_set(K, dense_fraction=p)
        else:
            assert oracle.resolve_dense_set(K, dense_fraction=p)[2] == kd


def test_dense_set_explicit():
    pi, K_s, K_d = oracle.resolve_dense_set(12, dense_cols=[11, 2, 7, 0])
    assert (K_s, K_d) == (8, 4)
    assert pi.tolist() == [1, 3, 4, 5, 6, 8, 9, 10, 0, 2, 7, 11]
    with pytest.raises(oracle.DenseSetError):
        oracle.resolve_dense_set(12, dense_cols=[1, 1, 2, 3])
    with pytest.raises(oracle.DenseSetError):
        oracle.resolve_dense_set(12, dense_cols=[12, 1, 2, 3])
    with pytest.raises(oracle.DenseSetError):
        oracle.resolve_dense_set(12, dense_cols=[1, 2])
    with pytest.raises(oracle.DenseSetError):
        oracle.resolve_dense_set(12, dense_fraction=1.5)


# --------------------------------------------------------------------------
# hand-worked examples
# --------------------------------------------------------------------------
def _golden_cases():
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_worked(case):
    K = case["K"]
    if "dense_cols" in case:
        pi, K_s, K_d = oracle.resolve_dense_set(K, dense_cols=case["dense_cols"])
    else:
        pi, K_s, K_d = oracle.resolve_dense_set(K, dense_fraction=case["dense_fraction"])
    e = case["expect"]
    assert pi.tolist() == e["pi"] and K_s == e["K_s"]
    if case["dtype"] == "f32":
        W = np.array(case["W"], dtype=np.float32)
        p = oracle.pack(W, DT_F32, pi, K_s)
        assert np.array_equal(p.vals, np.array(e["vals"], dtype=np.float32))
        assert np.array_equal(np.signbit(p.vals), np.signbit(np.array(e["vals"], dtype=np.float32)))
        assert np.array_equal(p.dense, np.array(e["dense"], dtype=np.float32).reshape(p.dense.shape))
        X = np.array(case["X"], dtype=np.float32)
        Y, B = oracle.linear_ref(X, DT_F32, p)
    elif case["dtype"] == "bf16":
        def bits(rows):
            return np.array([[int(v, 16) for v in row] for row in rows], dtype=np.uint16)
        W = bits(case["W_bits"])
        p = oracle.pack(W, DT_BF16, pi, K_s)
        assert np.array_equal(p.vals, bits(e["vals_bits"]))
        assert np.array_equal(p.dense, bits(e["dense_bits"]))
        X = synth.bf16_encode(np.array(case["X"], dtype=np.float64))
        Y, B = oracle.linear_ref(X, DT_BF16, p)
    else:
        W = np.array(case["W_codes"], dtype=np.uint8)
        p = oracle.pack(W, DT_FP8, pi, K_s)
        assert p.vals.tolist() == e["vals_codes"]
        assert p.dense.reshape(-1).tolist() == [c for row in e["dense_codes"] for c in row]
        X = synth.bf16_encode(np.array(case["X"], dtype=np.float64))
        Y, B = oracle.linear_ref(X, DT_BF16, p, scales=np.array(case["scales"], dtype=np.float32))
    assert p.meta.tolist() == e["meta"]
    assert p.mask.tolist() == e["mask"]
    assert np.array_equal(Y, np.array(e["Y"], dtype=np.float64))
    # the error scale of the pass rule, worked by hand over the pruned weights
    assert np.array_equal(B, np.array(e["B"], dtype=np.float64))


# --------------------------------------------------------------------------
# a2: the 2:4 choice, exhaustively
# --------------------------------------------------------------------------
def abs_order_key(bits, dtype):
    """Magnitude of each stored element, decoded by torch (not by the oracle):
    |value| in float64, with NaN above every number (the reading for NaN)."""
    b = np.ascontiguousarray(bits)
    if dtype == DT_F32:
        v = torch.from_numpy(b.astype(np.float32)).to(torch.float64)
    elif dtype == DT_BF16:
        v = torch.from_numpy(b.astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64)
    else:
        v = torch.from_numpy(b.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64)
    a = v.abs().numpy()
    return np.where(np.isnan(a), np.inf, a)


def _check_groups(W, dtype):
    """W[n, 4]: one group per row; compare oracle's choice with dominance on
    the decoded magnitudes."""
    pi = np.arange(4)
    p = oracle.pack(W, dtype, pi, 4)
    keys = abs_order_key(W, dtype)
    nib = p.meta[:, 0] & 0xF
    for n in range(W.shape[0]):
        i0, i1 = dominance_pair(keys[n].tolist())
        assert int(nib[n]) == (i0 | (i1 << 2)), (W[n], keys[n])
        assert p.mask[n].tolist() == [1 if t in (i0, i1) else 0 for t in range(4)]


def test_tie_break_exhaustive_small_ints():
    groups = np.array(list(itertools.product(range(-4, 5), repeat=4)), dtype=np.float64)
    groups[groups == 0] = 0.0
    _check_groups(groups.astype(np.float32), DT_F32)
    _check_groups(synth.bf16_encode(groups * 0.375), DT_BF16)
    _check_groups(synth.e4m3_encode(groups * 2.0), DT_FP8)
    # signed zeros in every position: -0 and +0 are equal magnitudes
    z = np.array(list(itertools.product([0.0, -0.0, 1.0, -1.0], repeat=4)), dtype=np.float32)
    _check_groups(z, DT_F32)


def test_tie_break_all_e4m3_code_pairs():
    a, b = np.meshgrid(np.arange(256), np.arange(256), indexing="ij")
    a = a.ravel().astype(np.uint8)
    b = b.ravel().astype(np.uint8)
    for patt in ((a, b, b, a), (a, a, b, b), (b, a, a, b)):
        W = np.stack(patt, axis=1)
        p = oracle.pack(W, DT_FP8, np.arange(4), 4)
        keys = abs_order_key(W, DT_FP8)
        # vectorised dominance: count for each candidate pair whether it dominates
        nib = (p.meta[:, 0] & 0xF).astype(np.int64)
        sel = np.zeros(W.shape[0], dtype=np.int64) - 1
        for P in itertools.combinations(range(4), 2):
            ok = np.ones(W.shape[0], dtype=bool)
            for i in P:
                for j in range(4):
                    if j in P:
                        continue
                    ok &= (keys[:, i] > keys[:, j]) | ((keys[:, i] == keys[:, j]) & (i < j))
            assert not np.any(ok & (sel >= 0))
            sel[ok] = P[0] | (P[1] << 2)
        assert np.all(sel >= 0)
        assert np.array_equal(sel, nib)


@pytest.mark.parametrize("dtype", [DT_BF16, DT_FP8])
def test_key_order_is_magnitude_order_every_code(dtype):
    """Over every bf16 bit pattern and every e4m3 code (NaN excluded), the
    oracle's key orders elements exactly as their magnitudes decoded by torch:
    sorted by key, |value| never decreases, and two codes share a key exactly
    when they share a magnitude (so +x and -x tie, and +0 ties -0)."""
    n = 65536 if dtype == DT_BF16 else 256
    codes = np.arange(n, dtype=np.uint32).astype(np.uint16 if dtype == DT_BF16 else np.uint8)
    t = torch.from_numpy(codes.view(np.int16) if dtype == DT_BF16 else codes)
    vals = t.view(torch.bfloat16 if dtype == DT_BF16 else torch.float8_e4m3fn).to(torch.float64).numpy()
    keep = ~np.isnan(vals)
    codes, a = codes[keep], np.abs(vals[keep])
    key = oracle.magnitude_key(codes, dtype)
    order = np.argsort(key, kind="stable")
    k, v = key[order], a[order]
    assert np.all(v[1:] >= v[:-1])
    assert np.array_equal(k[1:] == k[:-1], v[1:] == v[:-1])
    # every magnitude is held by exactly two codes (+ and -), both with one key
    assert np.all(np.unique(key, return_counts=True)[1] == 2)


def test_key_order_is_magnitude_order_fp32_sample():
    rng = np.random.default_rng(17)
    v = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 1e-40, 2000), [0.0, -0.0, 1e-45, -1e-45, 3e38]])
    v = np.concatenate([v, -v]).astype(np.float32)
    key = oracle.magnitude_key(v, DT_F32)
    a = np.abs(v.astype(np.float64))
    order = np.argsort(key, kind="stable")
    k, b = key[order], a[order]
    assert np.all(b[1:] >= b[:-1])
    assert np.array_equal(k[1:] == k[:-1], b[1:] == b[:-1])


# --------------------------------------------------------------------------
# invariants on random weights
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [DT_F32, DT_BF16, DT_FP8])
def test_two_of_four_and_round_trip(dtype):
    rng = np.random.default_rng(11)
    N, K = 24, 96
    W, s = synth.make_weight(N, K, dtype, rng)
    for D in (synth.tail_dense_set(K, 32), synth.random_dense_set(K, 20, 3), np.array([], dtype=np.int32)):
        pi, K_s, K_d = oracle.resolve_dense_set(K, dense_cols=D)
        p = oracle.pack(W, dtype, pi, K_s)
        # exactly two kept slots per group
        assert np.all(p.mask.reshape(N, -1, 4).sum(axis=2) == 2)
        Wr = oracle.unpack_bits(p)
        # pruned matrix: at most two nonzeros per group of the sparse region
        vals = oracle.decode_values(Wr, dtype)
        nz = (vals[:, pi[:K_s]] != 0).reshape(N, -1, 4).sum(axis=2)
        assert np.all(nz <= 2)
        # round trip against the mask applied to W (computed here, not by unpack)
        keep = np.ones((N, K), dtype=bool)
        keep[:, pi[:K_s]] = p.mask.astype(bool)
        zero = np.zeros((), dtype=W.dtype)
        expect = np.where(keep, W, zero)
        assert np.array_equal(expect.view(np.uint8), Wr.view(np.uint8))
        # idempotence: packing the pruned matrix gives the same packed form
        p2 = oracle.pack(Wr, dtype, pi, K_s)
        assert np.array_equal(p2.meta, p.meta) and np.array_equal(p2.mask, p.mask)


# --------------------------------------------------------------------------
# special cases that reduce to a library GEMM
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [DT_F32, DT_BF16, DT_FP8])
def test_fraction_one_is_dense_gemm(dtype):
    rng = np.random.default_rng(12)
    N, K, M = 40, 64, 3
    W, s = synth.make_weight(N, K, dtype, rng)
    X = synth.make_x(M, K, DT_F32 if dtype == DT_F32 else DT_BF16, rng)
    xdt = DT_F32 if dtype == DT_F32 else DT_BF16
    pi, K_s, K_d = oracle.resolve_dense_set(K, dense_fraction=1.0)
    assert K_s == 0
    p = oracle.pack(W, dtype, pi, K_s)
    Y, B = oracle.linear_ref(X, xdt, p, s)
    Wt = torch.from_numpy(oracle.decode_values(W, dtype))
    if s is not None:
        Wt = Wt * torch.from_numpy(s.astype(np.float64))[:, None]
    ref = torch.nn.functional.linear(torch.from_numpy(oracle.decode_values(X, xdt)), Wt).numpy()
    assert np.all(np.abs(Y - ref) <= 1e-12 * B + 1e-300)
    Yd, _ = oracle.dense_linear_ref(X, xdt, W, dtype, s)
    assert np.all(np.abs(Yd - ref) <= 1e-12 * B + 1e-300)


@pytest.mark.parametrize("dtype", [DT_F32, DT_FP8])
def test_fraction_zero_is_pure_two_four(dtype):
    rng = np.random.default_rng(13)
    N, K, M = 16, 64, 2
    W, s = synth.make_weight(N, K, dtype, rng)
    xdt = DT_F32 if dtype == DT_F32 else DT_BF16
    X = synth.make_x(M, K, xdt, rng)
    pi, K_s, K_d = oracle.resolve_dense_set(K, dense_fraction=0.0)
    p = oracle.pack(W, dtype, pi, K_s)
    Y, B = oracle.linear_ref(X, xdt, p, s)
    keys = oracle.magnitude_key(W, dtype)
    Wp = torch.tensor(prune_python(oracle.decode_values(W, dtype).tolist(), keys.tolist(), pi, K_s), dtype=torch.float64)
    if s is not None:
        Wp = Wp * torch.from_numpy(s.astype(np.float64))[:, None]
    ref = torch.nn.functional.linear(torch.from_numpy(oracle.decode_values(X, xdt)), Wp).numpy()
    assert np.all(np.abs(Y - ref) <= 1e-12 * B + 1e-300)


# --------------------------------------------------------------------------
# exact brute force over every dense set of a tiny layer
# --------------------------------------------------------------------------
def test_brute_force_every_dense_set_8x16():
    rng = np.random.default_rng(14)
    N, K, M = 8, 16, 2
    W = rng.integers(-6, 7, size=(N, K)).astype(np.float32)
    X = rng.integers(-5, 6, size=(M, K)).astype(np.float32)
    keys = oracle.magnitude_key(W, DT_F32).tolist()
    Wl = W.astype(np.float64).tolist()
    Xl = X.astype(np.float64).tolist()
    count = 0
    for kd in (0, 4, 8, 12, 16):
        for D in itertools.combinations(range(K), kd):
            pi, K_s, K_d = oracle.resolve_dense_set(K, dense_cols=list(D))
            p = oracle.pack(W, DT_F32, pi, K_s)
            Y, B = oracle.linear_ref(X, DT_F32, p)
            Wp = prune_python(Wl, keys, pi, K_s)
            for m in range(M):
                for n in range(N):
                    acc = bnd = 0.0
                    for k in range(K):
                        acc += Xl[m][k] * Wp[n][k]
                        bnd += abs(Xl[m][k] * Wp[n][k])
                    assert Y[m, n] == acc
                    assert B[m, n] == bnd
            count += 1
    assert count == 1 + 1820 + 12870 + 1820 + 1


def test_brute_force_e4m3_with_scales_and_bound():
    """e4m3 codes of small integers and halves, bf16 integer activations,
    per-channel scales: the layer output and its error scale by plain loops
    over weights pruned with the dominance rule on torch-decoded magnitudes
    (every product and sum is exact in float64, so equality is exact)."""
    rng = np.random.default_rng(18)
    N, K, M = 6, 24, 3
    vals = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, -0.5, -1.0, -2.0, -3.0, -4.0, -0.0],
                        dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    W = rng.choice(vals, size=(N, K))
    X = synth.bf16_encode(rng.integers(-7, 8, size=(M, K)).astype(np.float64))
    s = np.array([0.375, 1.0, 2.5, 0.0078125, 1.75, 3.0], dtype=np.float32)
    D = [0, 5, 6, 13, 14, 23, 2, 9]
    pi, K_s, _ = oracle.resolve_dense_set(K, dense_cols=D)
    Y, B = oracle.linear_ref(X, DT_BF16, oracle.pack(W, DT_FP8, pi, K_s), s)
    mag = abs_order_key(W, DT_FP8).tolist()
    wv = torch.from_numpy(W).view(torch.float8_e4m3fn).to(torch.float64).numpy().tolist()
    xv = torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy().tolist()
    for n in range(N):
        row = list(wv[n])
        for g in range(K_s // 4):
            cols = [int(pi[4 * g + t]) for t in range(4)]
            P = dominance_pair([mag[n][c] for c in cols])
            for t in range(4):
                if t not in P:
                    row[cols[t]] = 0.0
        for m in range(M):
            acc = bnd = 0.0
            for k in range(K):
                acc += xv[m][k] * row[k]
                bnd += abs(xv[m][k] * row[k])
            assert Y[m, n] == float(s[n]) * acc
            assert B[m, n] == float(s[n]) * bnd


def test_down_ref_brute_force_loops():
    """The down projection on float64 activations: output and error scale by
    plain loops over the pruned weights (dominance rule, scales applied after
    the sums); integer-valued inputs keep every sum exact."""
    rng = np.random.default_rng(19)
    H, I, M = 5, 16, 2
    vals = torch.tensor([0.0, 1.0, 2.0, 3.0, -1.0, -2.0, -3.0], dtype=torch.float32).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    Wd = rng.choice(vals, size=(H, I))
    A = rng.integers(-6, 7, size=(M, I)).astype(np.float64)
    sd = np.array([0.5, 1.25, 2.0, 0.125, 4.0], dtype=np.float32)
    D = [3, 4, 10, 15]
    pi, K_s, _ = oracle.resolve_dense_set(I, dense_cols=D)
    Y, B = oracle.down_ref(A, oracle.pack(Wd, DT_FP8, pi, K_s), sd)
    mag = abs_order_key(Wd, DT_FP8).tolist()
    wv = torch.from_numpy(Wd).view(torch.float8_e4m3fn).to(torch.float64).numpy().tolist()
    for n in range(H):
        row = list(wv[n])
        for g in range(K_s // 4):
            cols = [int(pi[4 * g + t]) for t in range(4)]
            P = dominance_pair([mag[n][c] for c in cols])
            for t in range(4):
                if t not in P:
                    row[cols[t]] = 0.0
        for m in range(M):
            acc = sum(A[m, k] * row[k] for k in range(I))
            bnd = sum(abs(A[m, k] * row[k]) for k in range(I))
            assert Y[m, n] == float(sd[n]) * acc
            assert B[m, n] == float(sd[n]) * bnd


# --------------------------------------------------------------------------
# permutation into the dense block leaves the output unchanged
# --------------------------------------------------------------------------
def test_gather_equals_contiguous_tail():
    rng = np.random.default_rng(15)
    N, K, M = 32, 128, 4
    W = rng.integers(-8, 9, size=(N, K)).astype(np.float32)
    X = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    D = synth.random_dense_set(K, 32, 7)
    pi, K_s, K_d = oracle.resolve_dense_set(K, dense_cols=D)
    Y1, _ = oracle.linear_ref(X, DT_F32, oracle.pack(W, DT_F32, pi, K_s))
    pi2, K_s2, _ = oracle.resolve_dense_set(K, dense_fraction=K_d / K)
    Y2, _ = oracle.linear_ref(X[:, pi], DT_F32, oracle.pack(W[:, pi], DT_F32, pi2, K_s2))
    assert np.array_equal(Y1, Y2)


def test_scale_is_per_output_channel():
    rng = np.random.default_rng(16)
    N, K, M = 8, 32, 2
    W, s = synth.make_weight(N, K, DT_FP8, rng)
    X = synth.make_x(M, K, DT_BF16, rng)
    pi, K_s, _ = oracle.resolve_dense_set(K, dense_fraction=0.25)
    p = oracle.pack(W, DT_FP8, pi, K_s)
    Y, _ = oracle.linear_ref(X, DT_BF16, p, s)
    Y1, _ = oracle.linear_ref(X, DT_BF16, p, None)
    assert np.array_equal(Y, Y1 * s.astype(np.float64)[None, :])
    # the scale is max|w|/448 of the unpruned row: every row holds a +-448 code
    assert np.all(np.max(oracle.magnitude_key(W, DT_FP8), axis=1) == 0x7E)


# --------------------------------------------------------------------------
# output-split form (dense rows | 2:4 rows)
# --------------------------------------------------------------------------
def test_dense_rows_resolution():
    rho, N_s, N_d = oracle.resolve_dense_rows(10, 8, dense_fraction=0.25)
    assert (N_s, N_d) == (7, 3) and rho.tolist() == list(range(10))  # round(2.5) = 3, half away from zero
    rho, N_s, N_d = oracle.resolve_dense_rows(6, 8, dense_rows=[4, 1])
    assert (N_s, N_d) == (4, 2) and rho.tolist() == [0, 2, 3, 5, 1, 4]
    rho, N_s, N_d = oracle.resolve_dense_rows(3, 6, dense_fraction=1.0)  # no sparse row: K need not be a multiple of 4
    assert (N_s, N_d) == (0, 3)
    for bad in ([6], [-1], [2, 2]):
        with pytest.raises(oracle.DenseSetError):
            oracle.resolve_dense_rows(6, 8, dense_rows=bad)
    with pytest.raises(oracle.DenseSetError):
        oracle.resolve_dense_rows(6, 6, dense_rows=[0])


@pytest.mark.parametrize("dtype", [DT_F32, DT_BF16, DT_FP8])
def test_rows_fraction_one_is_dense_gemm(dtype):
    rng = np.random.default_rng(41)
    N, K, M = 24, 64, 3
    W, s = synth.make_weight(N, K, dtype, rng)
    xdt = DT_F32 if dtype == DT_F32 else DT_BF16
    X = synth.make_x(M, K, xdt, rng)
    rho, N_s, _ = oracle.resolve_dense_rows(N, K, dense_fraction=1.0)
    Y, B = oracle.linear_rows_ref(X, xdt, oracle.pack_rows(W, dtype, rho, N_s), s)
    Wt = torch.from_numpy(oracle.decode_values(W, dtype))
    if s is not None:
        Wt = Wt * torch.from_numpy(s.astype(np.float64))[:, None]
    ref = torch.nn.functional.linear(torch.from_numpy(oracle.decode_values(X, xdt)), Wt).numpy()
    assert np.all(np.abs(Y - ref) <= 1e-12 * B + 1e-300)


@pytest.mark.parametrize("dtype", [DT_F32, DT_FP8])
def test_rows_fraction_zero_is_pure_two_four(dtype):
    rng = np.random.default_rng(42)
    N, K, M = 12, 32, 2
    W, s = synth.make_weight(N, K, dtype, rng)
    xdt = DT_F32 if dtype == DT_F32 else DT_BF16
    X = synth.make_x(M, K, xdt, rng)
    rho, N_s, _ = oracle.resolve_dense_rows(N, K, dense_fraction=0.0)
    Y, B = oracle.linear_rows_ref(X, xdt, oracle.pack_rows(W, dtype, rho, N_s), s)
    keys = oracle.magnitude_key(W, dtype)
    Wp = torch.tensor(prune_python(oracle.decode_values(W, dtype).tolist(), keys.tolist(), np.arange(K), K),
                      dtype=torch.float64)
    if s is not None:
        Wp = Wp * torch.from_numpy(s.astype(np.float64))[:, None]
    ref = torch.nn.functional.linear(torch.from_numpy(oracle.decode_values(X, xdt)), Wp).numpy()
    assert np.all(np.abs(Y - ref) <= 1e-12 * B + 1e-300)


def test_rows_split_column_by_column():
    """Each output column is either the dense product of its row or the
    input-split layer with no dense columns (pinned above) on that row."""
    rng = np.random.default_rng(43)
    N, K, M = 40, 96, 3
    W, s = synth.make_weight(N, K, DT_FP8, rng)
    X = synth.make_x(M, K, DT_BF16, rng)
    D = synth.random_dense_set(N, 9, 44)
    rho, N_s, _ = oracle.resolve_dense_rows(N, K, dense_rows=D)
    Y, _ = oracle.linear_rows_ref(X, DT_BF16, oracle.pack_rows(W, DT_FP8, rho, N_s), s)
    Yd, _ = oracle.dense_linear_ref(X, DT_BF16, W, DT_FP8, s)
    pi, K_s, _ = oracle.resolve_dense_set(K, dense_fraction=0.0)
    Ys, _ = oracle.linear_ref(X, DT_BF16, oracle.pack(W, DT_FP8, pi, K_s), s)
    dense = np.zeros(N, dtype=bool)
    dense[D] = True
    assert np.array_equal(Y[:, dense], Yd[:, dense])
    assert np.array_equal(Y[:, ~dense], Ys[:, ~dense])


def test_rows_brute_force_every_dense_row_set_6x8():
    rng = np.random.default_rng(45)
    N, K, M = 6, 8, 2
    W = rng.integers(-5, 6, size=(N, K)).astype(np.float32)
    X = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    keys = oracle.magnitude_key(W, DT_F32).tolist()
    Xl = X.astype(np.float64).tolist()
    count = 0
    for nd in range(N + 1):
        for D in itertools.combinations(range(N), nd):
            rho, N_s, _ = oracle.resolve_dense_rows(N, K, dense_rows=list(D))
            p = oracle.pack_rows(W, DT_F32, rho, N_s)
            Y, B = oracle.linear_rows_ref(X, DT_F32, p)
            for n in range(N):
                row = [float(v) for v in W[n]]
                if n not in D:
                    for g in range(K // 4):
                        P = dominance_pair([keys[n][4 * g + t] for t in range(4)])
                        for t in range(4):
                            if t not in P:
                                row[4 * g + t] = 0.0
                for m in range(M):
                    acc = bnd = 0.0
                    for k in range(K):
                        acc += Xl[m][k] * row[k]
                        bnd += abs(Xl[m][k] * row[k])
                    assert Y[m, n] == acc
                    assert B[m, n] == bnd
            count += 1
    assert count == 2 ** N


def test_rows_permutation_moves_outputs_only():
    """Moving a chosen row set into a contiguous tail (rows permuted) permutes
    the output columns the same way and changes nothing else."""
    rng = np.random.default_rng(46)
    N, K, M = 48, 64, 3
    W = rng.integers(-8, 9, size=(N, K)).astype(np.float32)
    X = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    D = synth.random_dense_set(N, 12, 47)
    rho, N_s, N_d = oracle.resolve_dense_rows(N, K, dense_rows=D)
    Y1, _ = oracle.linear_rows_ref(X, DT_F32, oracle.pack_rows(W, DT_F32, rho, N_s))
    rho2, N_s2, _ = oracle.resolve_dense_rows(N, K, dense_fraction=N_d / N)
    Y2, _ = oracle.linear_rows_ref(X, DT_F32, oracle.pack_rows(W[rho], DT_F32, rho2, N_s2))
    assert np.array_equal(Y1[:, rho], Y2)


def test_rows_pack_round_trip():
    rng = np.random.default_rng(48)
    N, K = 20, 64
    W, _ = synth.make_weight(N, K, DT_BF16, rng)
    D = synth.random_dense_set(N, 5, 49)
    rho, N_s, _ = oracle.resolve_dense_rows(N, K, dense_rows=D)
    p = oracle.pack_rows(W, DT_BF16, rho, N_s)
    U = oracle.unpack_rows_bits(p)
    assert np.array_equal(U[D], W[D])
    sp = np.setdiff1d(np.arange(N), D)
    kept = (U[sp] != 0) | (W[sp] == 0)
    assert np.all(kept.reshape(len(sp), K // 4, 4).sum(axis=2) >= 2)
    nz = (U[sp] != 0).reshape(len(sp), K // 4, 4).sum(axis=2)
    assert np.all(nz <= 2)
    assert np.array_equal(U[sp][U[sp] != 0], W[sp][U[sp] != 0])
    p2 = oracle.pack_rows(U, DT_BF16, rho, N_s)
    assert np.array_equal(p2.sparse.vals, p.sparse.vals) and np.array_equal(p2.sparse.meta, p.sparse.meta)


# --------------------------------------------------------------------------
# GLU block (gate/up output-split, SiLU * up, down input-split)
# --------------------------------------------------------------------------
def test_silu_matches_torch():
    x = np.concatenate([np.linspace(-60, 60, 2001), [-1e3, -80.0, 0.0, 1e-30, 80.0, 1e3]])
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    assert np.allclose(oracle.silu(x), ref, rtol=1e-15, atol=1e-300)


def _glu_weights(H, I, dtype, seed):
    rng = np.random.default_rng(seed)
    Wg, sg = synth.make_weight(I, H, dtype, rng)
    Wu, su = synth.make_weight(I, H, dtype, rng)
    Wd, sd = synth.make_weight(H, I, dtype, rng)
    X = synth.make_x(3, H, DT_BF16, rng)
    return X, Wg, sg, Wu, su, Wd, sd


def _torch_block(X, Wg, Wu, Wd, dtype, sg, su, sd):
    def w(Wb, s):
        t = torch.from_numpy(oracle.decode_values(Wb, dtype) if Wb.dtype != np.float64 else Wb)
        return t * torch.from_numpy(s.astype(np.float64))[:, None] if s is not None else t
    x = torch.from_numpy(oracle.decode_values(X, DT_BF16))
    g = torch.nn.functional.linear(x, w(Wg, sg))
    u = torch.nn.functional.linear(x, w(Wu, su))
    a = torch.nn.functional.silu(g) * u
    return torch.nn.functional.linear(a, w(Wd, sd)).numpy()


@pytest.mark.parametrize("dtype", [DT_BF16, DT_FP8])
def test_glu_all_dense_is_textbook_block(dtype):
    H, I = 64, 96
    X, Wg, sg, Wu, su, Wd, sd = _glu_weights(H, I, dtype, 51)
    r = oracle.glu_block_ref(X, DT_BF16, Wg, Wu, Wd, dtype, np.arange(I), sg, su, sd)
    ref = _torch_block(X, Wg, Wu, Wd, dtype, sg, su, sd)
    assert np.all(np.abs(r["Y"] - ref) <= 1e-12 * np.abs(ref).max() + 1e-300)


def test_glu_no_dense_index_is_pure_two_four_block():
    H, I, dtype = 32, 48, DT_FP8
    X, Wg, sg, Wu, su, Wd, sd = _glu_weights(H, I, dtype, 52)
    r = oracle.glu_block_ref(X, DT_BF16, Wg, Wu, Wd, dtype, [], sg, su, sd)

    def pruned(Wb, K):
        keys = oracle.magnitude_key(Wb, dtype).tolist()
        return np.array(prune_python(oracle.decode_values(Wb, dtype).tolist(), keys, np.arange(K), K))
    ref = _torch_block(X, pruned(Wg, H), pruned(Wu, H), pruned(Wd, I), dtype, sg, su, sd)
    assert np.all(np.abs(r["Y"] - ref) <= 1e-12 * np.abs(ref).max() + 1e-300)


def test_glu_permuted_block_equals_original():
    """Moving the chosen intermediate indices into a contiguous tail (gate/up
    rows and down columns permuted by rho) leaves the block output unchanged."""
    H, I, dtype = 64, 80, DT_FP8
    X, Wg, sg, Wu, su, Wd, sd = _glu_weights(H, I, dtype, 53)
    D = synth.random_dense_set(I, 20, 54)
    r1 = oracle.glu_block_ref(X, DT_BF16, Wg, Wu, Wd, dtype, D, sg, su, sd)
    rho = r1["rho"]
    tail = np.arange(I - len(D), I)
    r2 = oracle.glu_block_ref(X, DT_BF16, Wg[rho], Wu[rho], Wd[:, rho], dtype, tail, sg[rho], su[rho], sd)
    assert np.allclose(r2["A"], r1["A"][:, rho], rtol=0, atol=0)
    assert np.all(np.abs(r1["Y"] - r2["Y"]) <= 1e-12 * r1["B_Y"] + 1e-300)


# --------------------------------------------------------------------------
# SpenseGPT+ scores and dense index selection
# --------------------------------------------------------------------------

def test_scores_closed_form():
    """All-ones weights and constant calibration columns: every index scores
    2 H sqrt(T) |v| + H sqrt(sum_t a_ti^2)."""
    H, I, T = 8, 12, 5
    one = np.full((I, H), 0x3F80, dtype=np.uint16)           # bf16 1.0
    Wd = np.full((H, I), 0x3F80, dtype=np.uint16)
    X = np.full((T, H), 0x4000, dtype=np.uint16)             # bf16 2.0
    rng = np.random.default_rng(55)
    A = synth.make_x(T, I, DT_BF16, rng)
    a = oracle.decode_values(A, DT_BF16)
    s = oracle.glu_scores_ref(X, A, DT_BF16, one, one, Wd, DT_BF16)
    ref = 2 * H * np.sqrt(T) * 2.0 + H * np.sqrt((a * a).sum(axis=0))
    assert np.allclose(s, ref, rtol=1e-14, atol=0)


def test_scores_brute_force_loops_with_scales():
    H, I, T = 4, 6, 3
    rng = np.random.default_rng(56)
    Wg, sg = synth.make_weight(I, H, DT_FP8, rng)
    Wu, su = synth.make_weight(I, H, DT_FP8, rng)
    Wd, sd = synth.make_weight(H, I, DT_FP8, rng)
    X = synth.make_x(T, H, DT_BF16, rng)
    A = synth.make_x(T, I, DT_BF16, rng)
    s = oracle.glu_scores_ref(X, A, DT_BF16, Wg, Wu, Wd, DT_FP8, sg, su, sd)
    x = oracle.decode_values(X, DT_BF16).tolist()
    a = oracle.decode_values(A, DT_BF16).tolist()
    g, u, dn = (oracle.decode_values(w, DT_FP8).tolist() for w in (Wg, Wu, Wd))
    for i in range(I):
        tot = 0.0
        for j in range(H):
            hjj = sum(x[t][j] ** 2 for t in range(T))
            tot += abs(g[i][j] * float(sg[i])) * hjj ** 0.5 + abs(u[i][j] * float(su[i])) * hjj ** 0.5
        hii = sum(a[t][i] ** 2 for t in range(T))
        for n in range(H):
            tot += abs(dn[n][i] * float(sd[n])) * hii ** 0.5
        assert abs(s[i] - tot) <= 1e-12 * tot


def test_scores_follow_index_permutation():
    H, I, T = 16, 24, 7
    rng = np.random.default_rng(57)
    Wg, _ = synth.make_weight(I, H, DT_BF16, rng)
    Wu, _ = synth.make_weight(I, H, DT_BF16, rng)
    Wd, _ = synth.make_weight(H, I, DT_BF16, rng)
    X = synth.make_x(T, H, DT_BF16, rng)
    A = synth.make_x(T, I, DT_BF16, rng)
    p = rng.permutation(I)
    s = oracle.glu_scores_ref(X, A, DT_BF16, Wg, Wu, Wd, DT_BF16)
    sp = oracle.glu_scores_ref(X, A[:, p], DT_BF16, Wg[p], Wu[p], Wd[:, p], DT_BF16)
    assert np.allclose(sp, s[p], rtol=1e-15, atol=0)


def test_select_dense_rank_definition():
    """Top-k by the rank definition (count of strictly larger scores, plus equal
    scores at lower indices), brute force over small integer score vectors."""
    rng = np.random.default_rng(58)
    for _ in range(200):
        n = int(rng.integers(1, 12))
        sc = rng.integers(0, 4, size=n).astype(np.float64)
        k = int(rng.integers(0, n + 1))
        rank = [sum(1 for j in range(n) if sc[j] > sc[i] or (sc[j] == sc[i] and j < i)) for i in range(n)]
        want = sorted(i for i in range(n) if rank[i] < k)
        assert oracle.select_dense_ref(sc, k).tolist() == want
    assert oracle.select_dense_ref(np.array([1.0, 3.0, 3.0, 2.0, 3.0]), 2).tolist() == [1, 2]
    # infinities take their place in the order; NaN has none and is rejected
    assert oracle.select_dense_ref(np.array([1.0, np.inf, -np.inf, np.inf, 0.0]), 3).tolist() == [0, 1, 3]
    assert oracle.select_dense_ref(np.array([-np.inf, -np.inf, 0.0]), 2).tolist() == [0, 2]
    with pytest.raises(ValueError):
        oracle.select_dense_ref(np.array([1.0, np.nan, 0.0]), 1)


# --------------------------------------------------------------------------
# W8A8 (per-token e4m3 activations)
# --------------------------------------------------------------------------
def _e4m3_nearest_by_scan(v):
    """Brute force over all 256 codes: nearest finite value, ties to the even
    code, sign kept, saturating at 448 (independent of the oracle's search)."""
    v = float(np.float32(v))
    if v != v:
        return 0x7F
    a = min(abs(v), 448.0)
    best, best_d = None, None
    for c in range(0x7F):
        d = abs(oracle.decode_values(np.uint8(c), DT_FP8) - a)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best | (0x80 if np.signbit(np.float32(v)) else 0)


def test_e4m3_round_matches_torch_cast():
    """Inside the e4m3fn range the rounding is the library cast (round to nearest even)."""
    bf = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    rng = np.random.default_rng(41)
    v = np.concatenate([bf[np.isfinite(bf) & (np.abs(bf) <= 448.0)],
                        rng.uniform(-448, 448, 20000).astype(np.float32),
                        (rng.uniform(-1, 1, 5000) * 2.0 ** rng.integers(-14, -5, 5000)).astype(np.float32)])
    got = oracle.e4m3_round(v)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_e4m3_round_hand_cases_and_scan():
    # worked by hand: 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39):
    # the even code 0x38 wins; 1.1875 halfway between 0x39 and 1.25 (0x3A): 0x3A;
    # 2^-10 halfway between 0 and the smallest subnormal 2^-9 (0x01): 0x00;
    # 3 * 2^-10 halfway between 0x01 and 0x02: 0x02; 440 between 416 (0x7D) and 448 (0x7E): 0x7E
    cases = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02, 440.0: 0x7E,
             -1.0625: 0xB8, -2.0 ** -12: 0x80, 448.0: 0x7E, 449.0: 0x7E, 1e6: 0x7E, -1e6: 0xFE}
    for v, c in cases.items():
        assert int(oracle.e4m3_round(np.float32(v))) == c, v
    rng = np.random.default_rng(42)
    for v in np.concatenate([rng.uniform(-460, 460, 300), rng.uniform(-0.02, 0.02, 100)]).astype(np.float32):
        assert int(oracle.e4m3_round(v)) == _e4m3_nearest_by_scan(v), v


def test_e4m3_round_trip_every_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = oracle.decode_values(codes, DT_FP8).astype(np.float32)
    assert np.array_equal(oracle.e4m3_round(vals), codes)


def test_quantize_tokens_properties():
    rng = np.random.default_rng(43)
    X = synth.make_x(9, 300, DT_BF16, rng)
    X[4] = 0  # an all-zero token
    q, sx = oracle.quantize_tokens_ref(X, DT_BF16)
    Xv = oracle.decode_values(X, DT_BF16)
    amax = np.abs(Xv).max(axis=1)
    for m in range(9):
        if m == 4:
            assert sx[m] == 1.0 and not np.any(q[m] & 0x7F)
            continue
        assert sx[m] == np.float32(amax[m]) / np.float32(448.0)
        # the largest element of the token lands on +-448
        k = int(np.argmax(np.abs(Xv[m])))
        assert int(q[m, k]) & 0x7F == 0x7E
        # every code is within half a step of the exact quotient (e4m3 step at
        # magnitude a: 2^(floor(log2 a) - 3) for normals, 2^-9 for subnormals)
        t = Xv[m] / float(sx[m])
        a = np.maximum(np.abs(t), 2.0 ** -6)
        step = 2.0 ** (np.floor(np.log2(a)) - 3)
        err = np.abs(oracle.decode_values(q[m], DT_FP8) - t)
        assert np.all(err <= step / 2 * (1 + 1e-6))


@pytest.mark.parametrize("frac", [0.0, 0.25, 1.0])
def test_w8a8_equals_w8a16_when_tokens_are_representable(frac):
    """Tokens built as e4m3 values times a power of two whose largest magnitude
    is 448 times that power quantise without loss (s_x is the power of two, the
    quotients are exact e4m3 values); the W8A8 output then equals the W8A16
    output of the same X exactly (both sums are exact in float64)."""
    rng = np.random.default_rng(44)
    M, N, K = 5, 24, 256
    W, s = synth.make_weight(N, K, DT_FP8, rng)
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    codes = rng.choice(finite, size=(M, K))
    codes[:, 7] = 0x7E  # 448 in every token
    codes[1, 7] = 0xFE  # or -448
    e = rng.integers(-6, 3, size=M)
    Xv = oracle.decode_values(codes, DT_FP8) * (2.0 ** e)[:, None]
    X = torch.from_numpy(Xv.astype(np.float32)).to(torch.bfloat16).view(torch.uint16).numpy()
    assert np.array_equal(oracle.decode_values(X, DT_BF16), Xv)  # exact in bf16
    q, sx = oracle.quantize_tokens_ref(X, DT_BF16)
    assert np.array_equal(sx, (2.0 ** e).astype(np.float32))
    pi, K_s, _ = oracle.resolve_dense_set(K, dense_fraction=frac)
    P = oracle.pack(W, DT_FP8, pi, K_s)
    Y8, B8 = oracle.linear_w8a8_ref(q, sx, P, s)
    Y16, B16 = oracle.linear_ref(X, DT_BF16, P, s)
    assert np.array_equal(Y8, Y16) and np.array_equal(B8, B16)


def test_w8a8_tiny_brute_force_loops():
    """Triple loop over the decompressed weights with the scan quantiser above,
    scales included: equal to the oracle (integer-valued sums, exact)."""
    rng = np.random.default_rng(45)
    M, N, K = 3, 4, 16
    W, s = synth.make_weight(N, K, DT_FP8, rng)
    X = synth.make_x(M, K, DT_BF16, rng)
    D = [1, 6, 11, 12]
    pi, K_s, _ = oracle.resolve_dense_set(K, dense_cols=D)
    P = oracle.pack(W, DT_FP8, pi, K_s)
    q, sx = oracle.quantize_tokens_ref(X, DT_BF16)
    Y, B = oracle.linear_w8a8_ref(q, sx, P, s)
    Wbits = oracle.unpack_bits(P)
    Xv = oracle.decode_values(X, DT_BF16)
    for m in range(M):
        amax = max(abs(float(x)) for x in Xv[m])
        sxm = np.float32(amax) / np.float32(448.0) if amax > 0 else np.float32(1.0)
        qm = [_e4m3_nearest_by_scan(np.float32(Xv[m, k]) / sxm) for k in range(K)]
        assert qm == [int(c) for c in q[m]]
        for n in range(N):
            acc = bnd = 0.0
            for k in range(K):
                prod = float(oracle.decode_values(np.uint8(qm[k]), DT_FP8)) * float(
                    oracle.decode_values(Wbits[n, k], DT_FP8))
                acc += prod
                bnd += abs(prod)
            assert Y[m, n] == acc * (float(sxm) * float(np.float32(s[n])))
            assert B[m, n] == bnd * (float(sxm) * float(np.float32(s[n])))
