"""Checks on the gfx950 code the compiler emits for the HIP kernels (host-only).

A matrix instruction whose destination registers overlap its A or B source
registers gave wrong results on MI355X (seen with v_mfma_f32_16x16x32_bf16 and
VGPR accumulators, where the destination is a separate operand).  The kernels
now use only the structured-sparse instructions (v_smfmac_f32_16x16x64_bf16,
and v_smfmac_f32_16x16x128_fp8_fp8 for W8A8), whose destination is tied to
the accumulator; this test scans the emitted code for any overlap.  The code
is built with the flags of the product build.
"""

import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_dense_gemm_amd", "csrc")
SRCS = [os.path.join(CSRC, f) for f in ("spense_kernels.hip", "spense_tile.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


@pytest.fixture(scope="module")
def gfx950_asm():
    """gfx950 assembly of every kernel translation unit, built in parallel."""
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        from sparse_dense_gemm_amd.build import EXTRA, FLAGS

        flags = [f for f in FLAGS if f not in ("-fPIC", "-Wall", "-Wno-unused-function")]
        procs = []
        for i, src in enumerate(SRCS):
            out = os.path.join(d, f"k{i}.s")
            cmd = [HIPCC, *flags, *EXTRA.get(os.path.basename(src), []), "--cuda-device-only", "-S", src, "-o", out]
            procs.append((out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        text = []
        for out, pr in procs:
            _, err = pr.communicate()
            assert pr.returncode == 0, err[-2000:]
            with open(out) as f:
                text.append(f.read())
        return "\n".join(text)


def test_matrix_instructions_do_not_overwrite_their_sources(gfx950_asm):
    total, bad = 0, []
    for line in gfx950_asm.splitlines():
        m = re.match(r"\s+(v_s?mfmac?_\S+)\s+(.*)", line)
        if not m:
            continue
        ops = [o.strip() for o in m.group(2).split(";")[0].split(",")]
        total += 1
        if _regs(ops[0]) & (_regs(ops[1]) | _regs(ops[2])):
            bad.append(line.strip())
    assert total > 100
    assert not bad, bad[:5]


def test_no_packed_fp32_arithmetic(gfx950_asm):
    assert not re.search(r"\bv_pk_(add|mul|fma)_f32\b", gfx950_asm)


def test_both_regions_run_on_structured_sparse_instructions(gfx950_asm):
    # the 2:4 region and the dense region (as fixed-index products, index word
    # 0xEEEE4444) both use the structured-sparse instructions; no dense MFMA
    assert "v_smfmac_f32_16x16x64_bf16" in gfx950_asm
    assert "v_smfmac_f32_16x16x128_fp8_fp8" in gfx950_asm
    assert re.search(r"0xeeee4444", gfx950_asm, re.I)
    assert not re.search(r"\sv_mfma_", gfx950_asm)


def test_main_loops_keep_loads_in_flight(gfx950_asm):
    """The streaming kernels' main loops (those with structured-sparse
    instructions) wait on vector memory only with several loads still in
    flight: a wait for (almost) every outstanding load would drain the weight
    ring once per chunk."""
    labels = [(m.start(), m.group(1)) for m in re.finditer(r"^(_Z\w+):", gfx950_asm, re.M)]
    checked = 0
    for i, (pos, name) in enumerate(labels):
        if "linear_stream" not in name and "linear_tile" not in name:
            continue
        body = gfx950_asm[pos:labels[i + 1][0] if i + 1 < len(labels) else len(gfx950_asm)]
        loops, cur = {}, None
        for line in body.splitlines():
            if line.startswith(".LBB"):
                hm = re.search(r"Header=(\w+) Depth=1", line)
                cur = line.split(":")[0][1:] if "Loop Header: Depth=1" in line else (hm.group(1) if hm else None)
            if cur:
                d = loops.setdefault(cur, {"smf": 0, "vm": []})
                d["smf"] += "v_smfmac" in line
                w = re.search(r"s_waitcnt vmcnt\((\d+)\)", line)
                if w:
                    d["vm"].append(int(w.group(1)))
        main = max(loops.values(), key=lambda v: v["smf"], default=None)
        if not main or not main["vm"]:
            continue
        checked += 1
        if "linear_tile" in name:
            # the LDS-staged kernel waits once per stage, for its own copies of
            # that stage only: the copies of the NS - 2 later stages stay in
            # flight (none with a two-stage ring)
            m = re.search(r"I([ht])Lb([01])ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELb[01]E", name)
            wt, a8, wr, wm, r, t, ns = m.group(1), int(m.group(2)), *map(int, m.groups()[2:])
            nwv = wr * wm
            copies = (wr * r // nwv) * (2 if wt == "h" else 3) + (wm * t // nwv) * (2 if a8 else 4)
            assert set(main["vm"]) == {(ns - 2) * copies}, (name[:90], sorted(set(main["vm"])))
        else:
            assert min(main["vm"]) >= 4, (name[:90], sorted(set(main["vm"])))
    assert checked > 40


def _main_loop(body):
    """Lines of the depth-1 loop with the most structured-sparse instructions."""
    loops, cur = {}, None
    for line in body.splitlines():
        if line.startswith(".LBB"):
            hm = re.search(r"Header=(\w+) Depth=1", line)
            cur = line.split(":")[0][1:] if "Loop Header: Depth=1" in line else (hm.group(1) if hm else None)
        if cur:
            loops.setdefault(cur, []).append(line)
    return max(loops.values(), key=lambda ls: sum("v_smfmac" in x for x in ls), default=[])


def test_weights_read_once_stream_non_temporally(gfx950_asm):
    """Kernels that read each weight byte once (the decode kernels and the
    streaming kernels built for one m-group, template flag true) load the
    weight units with the non-temporal hint; the streaming kernels built for
    several m-groups (flag false), which re-read their weights from L2, do
    not."""
    labels = [(m.start(), m.group(1)) for m in re.finditer(r"^(_Z\w+):", gfx950_asm, re.M)]
    seen = {"decode": 0, "nt": 0, "default": 0}
    for i, (pos, name) in enumerate(labels):
        body = gfx950_asm[pos:labels[i + 1][0] if i + 1 < len(labels) else len(gfx950_asm)]
        loop = _main_loop(body)
        if "linear_decode" in name:
            loads = [x for x in loop if re.search(r"\sglobal_load_dwordx4\s", x)]
            assert loads and all(x.rstrip().endswith(" nt") for x in loads), (name[:90], loads[:3])
            seen["decode"] += 1
        elif "linear_tile" in name:
            # weight units and index blocks are copied into LDS with the
            # non-temporal hint in the one-m-group build, activations never
            loads = [x for x in body.splitlines() if re.search(r"\sbuffer_load_dword\S*\s.*\slds\b", x)]
            nt = [x for x in loads if re.search(r"\snt\b", x)]
            if "Lb1EEEv" in name:
                assert loads and nt and len(nt) < len(loads), name[:90]
                seen["nt"] += 1
            else:
                assert loads and not nt, (name[:90], nt[:3])
                seen["default"] += 1
        elif "linear_stream" in name:
            loads = [x for x in loop if re.search(r"\sbuffer_load_dwordx4\s", x)]
            nt = [x for x in loads if re.search(r"\snt\b", x)]
            if "Lb1EEEv" in name:  # last template argument (the one-m-group flag) true
                assert nt, name[:90]
                seen["nt"] += 1
            else:
                assert loads and not nt, (name[:90], nt[:3])
                seen["default"] += 1
    assert seen["decode"] >= 8 and seen["nt"] >= 20 and seen["default"] >= 40, seen


def test_decode_contiguous_staging_waits_only_for_its_copies(gfx950_asm):
    """The decode kernels on contiguous activations copy them into LDS with
    direct-to-LDS loads issued before the weight ring, then wait with the
    ring still in flight: the vector-memory wait before the first barrier
    must leave outstanding no more loads than were issued after the last
    copy (the counter retires in order, so every copy has then landed), and
    at least one (the ring is not drained)."""
    labels = [(m.start(), m.group(1)) for m in re.finditer(r"^(_Z\w+):", gfx950_asm, re.M)]
    checked = 0
    for i, (pos, name) in enumerate(labels):
        # template arguments end with (gather, swizzled rows): contiguous = gather false
        if "linear_decode" not in name or not re.search(r"Lb0ELb[01]EEEv", name):
            continue
        body = gfx950_asm[pos:labels[i + 1][0] if i + 1 < len(labels) else len(gfx950_asm)]
        copies = after = 0
        wait = None
        for line in body.splitlines():
            t = line.strip()
            if t.startswith("s_barrier"):
                break
            if re.search(r"^buffer_load_dword\S*\s.*\slds\b", t):
                assert after == 0, (name[:90], "a copy after a weight load")
                copies += 1
            elif re.match(r"(global|buffer)_load", t):
                after += 1
            w = re.search(r"s_waitcnt vmcnt\((\d+)\)", t)
            if w:
                wait = int(w.group(1))
        assert copies >= 1 and wait is not None, name[:90]
        assert 1 <= wait <= after, (name[:90], wait, after)
        checked += 1
    assert checked >= 16
