"""The batch-1 GEMV's streaming loops keep their loads in flight: compiled for gfx950 (hipcc on the
host, no GPU), each loop that holds the weight loads must wait only for the older register set
(s_waitcnt vmcnt(N) with N > 0), never for every load in flight. A vmcnt(0) there halves the loads
the kernel keeps in flight; it appeared once when a second copy of the loops was added to the kernel."""
import collections
import os
import re
import shutil
import subprocess

import pytest

from conftest import ROOT

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SRC = os.path.join(ROOT, "bit_plane_weight_amd", "csrc", "bpw_gemv.hip")


def loop_bodies(asm: str) -> dict:
    cur, blocks = None, collections.defaultdict(list)
    for line in asm.split("\n"):
        m = re.match(r"^(\.LBB\d+_\d+|; %bb\.\d+):(.*)$", line)
        if m:
            c = m.group(2)
            h = re.search(r"Header=BB(\d+_\d+)", c)
            if "Loop Header" in c and m.group(1).startswith(".LBB"):
                cur = "BB" + m.group(1).split("LBB")[1]
            elif h:
                cur = "BB" + h.group(1)
            else:
                cur = None
            continue
        if cur and line.startswith("\t") and not line.strip().startswith(";"):
            blocks[cur].append(line.strip())
    return blocks


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc not installed")
@pytest.mark.parametrize("src", [SRC, os.path.join(ROOT, "bit_plane_weight_amd", "csrc", "bpw_bytelane.hip")],
                         ids=["bitserial", "bytelane"])
def test_streaming_loops_wait_only_for_the_older_loads(tmp_path, src):
    """Both batch-1 kernels (the bit-serial select and the byte-lane select share the tile code)."""
    out = tmp_path / "gemv.s"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-S", "--cuda-device-only",
                    src, "-o", str(out)], check=True, capture_output=True)
    loops = {k: b for k, b in loop_bodies(out.read_text()).items()
             if sum("buffer_load_dwordx4" in x for x in b) >= 4}
    # the 2560-column loop (2 x 5 beat loads), the 6912-column loop (2 x 4) and the generic K = 2 one
    assert sorted(sum("buffer_load_dwordx4" in x for x in b) for b in loops.values()) == [4, 8, 10], loops.keys()
    for name, body in loops.items():
        waits = [int(m.group(1)) for x in body if (m := re.search(r"vmcnt\((\d+)\)", x))]
        assert waits and min(waits) > 0, f"loop {name}: vmcnt waits {waits}"


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc not installed")
def test_token_kernel_loops_wait_only_for_the_older_loads(tmp_path):
    """The same property for the 2-, 3- and 4-token kernels of the grouped small batch: per kernel one
    2560-column loop (2 x 5 beat loads) and one 6912-column loop (2 x 4), waits never vmcnt(0)."""
    out = tmp_path / "tokens.s"
    src = os.path.join(ROOT, "bit_plane_weight_amd", "csrc", "bpw_gemv_tokens.hip")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-S", "--cuda-device-only",
                    src, "-o", str(out)], check=True, capture_output=True)
    kernels = re.split(r"\n(?=_ZN3bpw18gemv_tokens_kernel)", out.read_text())[1:]
    assert len(kernels) == 3
    for k in kernels:
        loops = {n: b for n, b in loop_bodies(k).items() if sum("buffer_load_dwordx4" in x for x in b) >= 4}
        assert sorted(sum("buffer_load_dwordx4" in x for x in b) for b in loops.values()) == [8, 10], loops.keys()
        for name, body in loops.items():
            waits = [int(m.group(1)) for x in body if (m := re.search(r"vmcnt\((\d+)\)", x))]
            assert waits and min(waits) > 0, f"loop {name}: vmcnt waits {waits}"


def basic_blocks(asm: str) -> dict:
    blk, blocks = None, {}
    for line in asm.split("\n"):
        m = re.match(r"^(\.LBB\d+_\d+|; %bb\.\d+):", line)
        if m:
            blk = m.group(1)
            blocks[blk] = []
            continue
        if blk and line.startswith("\t") and not line.strip().startswith(";"):
            blocks[blk].append(line.strip())
    return blocks


def successors(blocks: dict) -> dict:
    """Control-flow successors of each basic block: its branch targets, and the next block unless it ends
    in an unconditional branch or the end of the program."""
    names, succ = list(blocks), {}
    for i, n in enumerate(names):
        body, out = blocks[n], []
        for x in body:
            m = re.match(r"s_c?branch\w*\s+(\.LBB\d+_\d+)", x)
            if m:
                out.append(m.group(1))
        last = body[-1] if body else ""
        if i + 1 < len(names) and not last.startswith("s_branch ") and not last.startswith("s_endpgm"):
            out.append(names[i + 1])
        succ[n] = out
    return succ


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc not installed")
def test_grouped_small_batch_stream_waits_only_for_the_older_loads(tmp_path):
    """The grouped matrix-core small batch: after every weight-beat load (the
    non-temporal 16-byte loads), each control-flow path reaches a matrix-core instruction before any wait
    that drains the vector-memory counter, so the beats a step issues for the next step stay in flight
    while the current step is decoded and multiplied. A path may end at a barrier instead: the beats a
    pass issues before staging its operands are waited for with the operands. A per-lane guard on the
    operand staging once left a load unwaited, and the compiler put waits for every load in flight into
    this loop. The paths are followed through the control flow because the compiler may put a step's
    loads and its matrix-core instructions in different basic blocks."""
    out = tmp_path / "sb.s"
    src = os.path.join(ROOT, "bit_plane_weight_amd", "csrc", "bpw_small_batch.hip")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-S", "--cuda-device-only",
                    src, "-o", str(out)], check=True, capture_output=True)
    kernels = re.split(r"\n(?=_ZN3bpw36gemm_small_batch_mfma_grouped_kernel)", out.read_text())[1:]
    assert len(kernels) == 1
    for kernel in kernels:
        kernel = kernel.split(".Lfunc_end")[0]
        blocks = basic_blocks(kernel)
        succ = successors(blocks)
        beat = lambda x: x.startswith("buffer_load_dwordx4") and x.endswith(" nt")
        assert sum(sum(beat(x) for x in b) for b in blocks.values()) >= 8, "no streaming loop found"
        assert sum(sum("v_mfma" in x for x in b) for b in blocks.values()) >= 16, "no matrix-core step found"

        def first_event(name, start):
            """'mfma', 'barrier' or 'end' on every path from instruction `start` of block `name`, or the
            block where a drain comes first."""
            seen, todo = set(), [(name, start)]
            while todo:
                n, i = todo.pop()
                stop = False
                for x in blocks[n][i:]:
                    if "v_mfma" in x or x.startswith("s_barrier") or x.startswith("s_endpgm"):
                        stop = True
                        break
                    if re.search(r"vmcnt\(0\)", x):
                        return n
                if not stop:
                    for m in succ[n]:
                        if m not in seen:
                            seen.add(m)
                            todo.append((m, 0))
            return None

        for name, body in blocks.items():
            loads = [i for i, x in enumerate(body) if beat(x)]
            if loads:
                bad = first_event(name, loads[-1] + 1)
                assert bad is None, f"beats loaded in {name}: a wait in {bad} drains them before the next step"


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc not installed")
def test_kernel_arguments_preloaded_except_the_quantiser(tmp_path):
    """The build preloads kernel arguments into SGPRs for the kernel files: the descriptor of a kernel
    whose arguments are pointers (the grouped GEMV, the grouped small batch) has a preload length, and
    its code starts with the compiler's fallback that loads them itself where the firmware does not.
    (Arguments passed as a structure by value are not preloaded.) The quantiser is built without it,
    as it measured slower with it."""
    from bit_plane_weight_amd import build as bpw_build
    for name, kernel, preloaded in (("bpw_gemv.hip", "gemv_bitserial_kernel", True),
                                    ("bpw_small_batch.hip", "gemm_small_batch_mfma_grouped_kernel", True),
                                    ("bpw_quantize.hip", "quantize_kernel", False)):
        src = os.path.join(ROOT, "bit_plane_weight_amd", "csrc", name)
        out = tmp_path / (name + ".s")
        flags = [f for f in bpw_build.flags_for(src) if f != "-fPIC"]
        subprocess.run([HIPCC, *flags, "-S", "--cuda-device-only", src, "-o", str(out)], check=True,
                       capture_output=True)
        blocks = re.findall(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", out.read_text(), re.S)
        lengths = [int(re.search(r"\.amdhsa_user_sgpr_kernarg_preload_length\s+(\d+)", b).group(1))
                   for k, b in blocks if kernel in k]
        assert len(lengths) == 1, (name, [k for k, _ in blocks])
        assert (lengths[0] > 0) == preloaded, (name, lengths)
