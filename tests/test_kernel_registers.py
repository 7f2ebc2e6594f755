"""The MFMA kernels' tile loops stay free of register spills.

Each kernel runs at two waves per SIMD, so a wave has 256 registers; values
that live across a whole work item may be spilled, but a spill reload inside a
tile loop is a vector-memory access that waits together with the loop's own
loads (and, after global stores, with those).  This compiles the two kernel
files to gfx950 assembly with the library's build flags and checks that no
basic block of an innermost loop (the tile loops) touches scratch memory.
CPU only: hipcc cross-compiles.
"""
import concurrent.futures
import os
import re
import subprocess

import pytest

from block_sparse_draft_amd import build as Bld

KERNELS = {
    "fwd_bf16.hip": ["fwd_bf16_kernel"],
    "bwd_bf16.hip": ["bwd_kv_kernel", "bwd_dq_kernel"],
}


def _assembly(src: str) -> str:
    try:
        cc = Bld.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    cmd = [cc] + Bld._flags() + Bld.EXTRA_FLAGS.get(src, []) + [
        "--cuda-device-only", "-S", os.path.join(Bld.CSRC, src), "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stdout


def _innermost_loop_ops(asm: str, kernel: str):
    """Instructions of every basic block inside an innermost loop of `kernel`,
    from the loop comments LLVM writes into the assembly; None if absent."""
    lines = asm.split("\n")
    sym = re.compile(r"^_Z\w*" + kernel + r"\w*:")
    start = next((i for i, l in enumerate(lines) if sym.match(l)), None)
    if start is None:
        return None
    end = next(i for i in range(start, len(lines)) if "s_endpgm" in lines[i])
    lines = lines[start:end]
    # headers of innermost loops: a header line with no "Child Loop" below it before the next block
    heads = set()
    for i, l in enumerate(lines):
        if "Loop Header: Depth=" in l:
            j = i + 1
            child = False
            while j < len(lines) and lines[j].lstrip().startswith(";"):
                child |= "Child Loop" in lines[j]
                j += 1
            if not child:
                lab = next((lines[k].split(":")[0] for k in range(i, -1, -1) if lines[k].startswith(".LBB")), None)
                if lab:
                    heads.add(lab[2:])
    if not heads:
        return None
    blocks = [i for i, l in enumerate(lines) if re.match(r"^(\.LBB\d+_\d+):|^; %bb\.\d+:", l)]
    ops = {}
    for bi, i in enumerate(blocks):
        ctx = " ".join(lines[i:i + 3])
        hit = [h for h in heads if ".L" + h + ":" in ctx or "Header=" + h + " " in ctx + " "]
        if not hit:
            continue
        stop = blocks[bi + 1] if bi + 1 < len(blocks) else len(lines)
        ops.setdefault(hit[0], []).extend(
            t.strip().split()[0] for t in lines[i:stop] if t.strip() and not t.strip().startswith((";", ".")))
    return ops


@pytest.fixture(scope="module")
def assembly():
    with concurrent.futures.ThreadPoolExecutor(len(KERNELS)) as ex:
        return dict(zip(KERNELS, ex.map(_assembly, KERNELS)))


@pytest.mark.parametrize("src,kernel", [(s, k) for s, ks in KERNELS.items() for k in ks])
def test_tile_loops_have_no_spill_accesses(assembly, src, kernel):
    loops = _innermost_loop_ops(assembly[src], kernel)
    if not loops:
        pytest.skip(f"no loop structure comments for {kernel} in this compiler's output")
    tile_loops = {h: ops for h, ops in loops.items() if "v_mfma_f32_32x32x16_bf16" in ops}
    assert tile_loops, f"{kernel}: no innermost loop with MFMAs found"
    for head, ops in tile_loops.items():
        spills = [op for op in ops if op.startswith("scratch_")]
        assert not spills, f"{kernel}: {len(spills)} scratch accesses in the tile loop {head}"


def test_loop_parser_sees_a_spill_in_a_loop():
    """The parser on a hand-written fragment: a spill reload in an innermost
    loop's body block is found, one in the enclosing loop is not counted."""
    asm = "\n".join([
        "_ZN3skv12_GLOBAL__N_16kernelEv: ; @x",
        ".LBB0_1:                ; =>This Loop Header: Depth=1",
        "                        ;     Child Loop BB0_2 Depth 2",
        "\tscratch_load_dword v1, off, off",
        ".LBB0_2:                ;   Parent Loop BB0_1 Depth=1",
        "                        ; =>  This Inner Loop Header: Depth=2",
        "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]",
        "; %bb.3:                ;   in Loop: Header=BB0_2 Depth=2",
        "\tscratch_load_dwordx4 v[8:11], off, off offset:16",
        "\ts_cbranch_scc1 .LBB0_2",
        "; %bb.4:                ;   in Loop: Header=BB0_1 Depth=1",
        "\ts_branch .LBB0_1",
        "\ts_endpgm",
    ])
    loops = _innermost_loop_ops(asm, "kernel")
    assert list(loops) == ["BB0_2"]
    assert loops["BB0_2"] == ["v_mfma_f32_32x32x16_bf16", "scratch_load_dwordx4", "s_cbranch_scc1"]
