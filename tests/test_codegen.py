"""Generated-code checks of the MFMA kernels (CPU only: needs hipcc, no GPU).

The kernels issue their MFMAs as inline asm (the accumulator tied in and out),
so the compiler inserts no wait states around them: the code itself has to
keep every MFMA's operands and results apart from other instructions.  These
tests compile the library's kernel sources to gfx950 assembly with the
build's flags and check, over each kernel's control-flow graph (loop back
edges included):

* no vector ALU instruction writes a register an MFMA reads (its A, B, C or
  scale operands) within the 6 issue slots before it (the hardware needs 2);
* no instruction other than an MFMA reads or writes an MFMA's result
  registers within the 18 issue slots after it (the longest MFMA here, 16
  passes, needs fewer);

counting ``s_nop N`` as N + 1 slots.  A synthetic listing with one planted
violation of each kind checks the checker.

The kernels' LDS rings count their loads themselves (the loads are inline
asm, which the compiler does not track, so each wait is the kernel's own
``s_waitcnt vmcnt(N)``).  A vector-memory wait the compiler adds inside a
loop (for loads of its own it believes still pending) waits for every load
in flight, the ring's prefetches included: a further check finds none in
any loop of the GEMM kernels (a synthetic listing checks it too).
"""
import os
import re
import subprocess

import pytest

from dense_gemm_08_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "dense_gemm_08_amd", "csrc")

BEFORE = 6    # issue slots checked before an MFMA for writes of its sources
AFTER = 18    # issue slots checked after an MFMA for uses of its results

pytestmark = pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not available")


# ---------------------------------------------------------------- parsing --

_REG = re.compile(r"^([va])\[(\d+):(\d+)\]$|^([va])(\d+)$")


def regs(tok: str):
    m = _REG.match(tok.strip())
    if not m:
        return set()
    if m.group(1):
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {(m.group(4), int(m.group(5)))}


def operands(ins: str):
    parts = ins.split(None, 1)
    if len(parts) < 2:
        return []
    return [t for t in re.split(r"[\s,]+", parts[1]) if t]


def is_mfma(ins: str) -> bool:
    return ins.startswith("v_mfma")


def slots(ins: str) -> int:
    if ins.startswith("s_nop"):
        return int(ins.split()[1], 0) + 1
    return 1


def kernels(asm: str):
    """{kernel name: [(label or None, instruction), ...]} for each kernel."""
    out, cur = {}, None
    for line in asm.split("\n"):
        s = line.split(";")[0].rstrip()
        m = re.match(r"^(_Z\S*kernel\S*):", s)
        if m:
            cur = out.setdefault(m.group(1), [])
            continue
        if cur is None:
            continue
        t = s.strip()
        if re.match(r"^\.Lfunc_end", t):
            cur = None
            continue
        if not t or t.startswith("."):
            if t.endswith(":") and t.startswith(".LBB"):
                cur.append((t[:-1], None))
            continue
        if t.endswith(":"):
            continue
        cur.append((None, t))
    return out


def cfg(items):
    """Basic blocks of a kernel: (instructions, successor block indices)."""
    blocks, labels, cur = [], {}, []
    for label, ins in items:
        if label is not None:
            if cur or blocks:
                blocks.append(cur)
                cur = []
            labels[label] = len(blocks)
            continue
        cur.append(ins)
        if ins.startswith(("s_branch", "s_cbranch", "s_endpgm")):
            blocks.append(cur)
            cur = []
    blocks.append(cur)
    succ = []
    for b, ins_list in enumerate(blocks):
        s = []
        last = ins_list[-1] if ins_list else ""
        if last.startswith(("s_branch", "s_cbranch")):
            s.append(labels[last.split()[1]])
        if not last.startswith(("s_branch", "s_endpgm")) and b + 1 < len(blocks):
            s.append(b + 1)
        succ.append(s)
    pred = [[] for _ in blocks]
    for b, s in enumerate(succ):
        for t in s:
            pred[t].append(b)
    return blocks, succ, pred


def walk(blocks, nxt, b, i, budget, forward):
    """Instructions within `budget` issue slots after (forward) or before
    instruction i of block b, over all paths."""
    seen = set()
    stack = [(b, i, budget)]
    while stack:
        b, i, left = stack.pop()
        ins_list = blocks[b]
        rng = range(i + 1, len(ins_list)) if forward else range(i - 1, -1, -1)
        for k in rng:
            if left <= 0:
                break
            yield ins_list[k]
            left -= slots(ins_list[k])
        else:
            for nb in nxt[b]:
                start = -1 if forward else len(blocks[nb])
                key = (nb, left)
                if left > 0 and key not in seen:
                    seen.add(key)
                    stack.append((nb, start, left))


def check(asm: str):
    """List of hazard descriptions found in the assembly text."""
    bad = []
    for name, items in kernels(asm).items():
        blocks, succ, pred = cfg(items)
        for b, ins_list in enumerate(blocks):
            for i, ins in enumerate(ins_list):
                if not is_mfma(ins):
                    continue
                ops = operands(ins)
                dst = regs(ops[0])
                src = set()
                for t in ops[1:]:
                    src |= regs(t)
                for p in walk(blocks, pred, b, i, BEFORE, forward=False):
                    if p.startswith("v_") and not is_mfma(p):
                        po = operands(p)
                        if po and regs(po[0]) & src:
                            bad.append("%s: %r writes a source of %r" % (name, p, ins))
                for n in walk(blocks, succ, b, i, AFTER, forward=True):
                    if is_mfma(n):
                        continue
                    used = set()
                    for t in operands(n):
                        used |= regs(t)
                    if used & dst:
                        bad.append("%s: %r touches the result of %r" % (name, n, ins))
    return list(dict.fromkeys(bad))  # one entry per pair (several paths may find it)


def compile_asm(src: str, out: str) -> str:
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [build.HIPCC] + flags + ["--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"),
                                   "-I", CSRC, os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    with open(out) as f:
        return f.read()


# ------------------------------------------------------------------ tests --

SYNTHETIC = """
_Zsynthetic_kernel:
	v_mov_b32 v4, 0
	v_mfma_f32_16x16x32_f16 a[0:3], v[4:7], v[8:11], a[0:3]
.LBB0_1:
	s_nop 7
	v_mfma_f32_16x16x32_f16 a[4:7], v[12:15], v[16:19], a[4:7]
	v_accvgpr_read_b32 v20, a5
	s_cbranch_scc1 .LBB0_1
	s_endpgm
.Lfunc_end0:
"""


def test_checker_finds_planted_hazards():
    found = check(SYNTHETIC)
    # v4 written just before the first MFMA reads it; a5 read right after
    # the second MFMA writes it
    assert any("writes a source" in f and "v_mov_b32 v4" in f for f in found), found
    assert any("touches the result" in f and "a5" in f for f in found), found
    assert len(found) == 2, found
    # the same listing with the hazards spaced out is clean
    spaced = SYNTHETIC.replace("\tv_mov_b32 v4, 0\n", "\tv_mov_b32 v4, 0\n\ts_nop 7\n")
    spaced = spaced.replace("\tv_accvgpr_read_b32 v20, a5\n",
                            "\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\tv_accvgpr_read_b32 v20, a5\n")
    assert check(spaced) == [], check(spaced)


def test_back_edge_is_followed():
    # the loop's last instruction writes a source of the loop's first MFMA:
    # only the back edge connects them
    asm = """
_Zloop_kernel:
.LBB0_1:
	v_mfma_f32_16x16x32_f16 a[0:3], v[4:7], v[8:11], a[0:3]
	s_nop 7
	s_nop 7
	s_nop 7
	v_add_u32_e32 v8, 1, v8
	s_cbranch_scc1 .LBB0_1
	s_endpgm
.Lfunc_end0:
"""
    found = check(asm)
    assert len(found) == 1 and "v_add_u32_e32 v8" in found[0], found


@pytest.mark.parametrize("src", ["dense_gemm.hip", "gemm_mx.hip", "ladder.hip"])
def test_library_kernels_keep_mfma_operands_apart(src, tmp_path):
    asm = compile_asm(src, str(tmp_path / (src + ".s")))
    ks = kernels(asm)
    assert ks, "no kernels found in the generated code"
    n_mfma = sum(1 for items in ks.values() for _, ins in items if ins and is_mfma(ins))
    assert n_mfma > 0
    bad = check(asm)
    assert not bad, "\n".join(bad[:20])


# ------------------------------------------- compiler waits in the rings --

def gemm_functions(asm: str):
    """{function name: [(label or None, instruction, from inline asm)]} for
    every function whose name contains "gemm" (the tiled and small-output
    kernels)."""
    out, cur, in_asm = {}, None, False
    for line in asm.split("\n"):
        if ";;#ASMSTART" in line:
            in_asm = True
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            continue
        s = line.split(";")[0].rstrip()
        m = re.match(r"^(_Z\S*gemm\S*):", s)
        if m:
            cur = out.setdefault(m.group(1), [])
            continue
        if cur is None:
            continue
        t = s.strip()
        if t.startswith(".Lfunc_end"):
            cur = None
            continue
        if t.startswith(".LBB") and t.endswith(":"):
            cur.append((t[:-1], None, False))
            continue
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        cur.append((None, t, in_asm))
    return out


def compiler_waits_in_loops(asm: str):
    """The compiler's own vector-memory waits in blocks on a cycle."""
    found = []
    for name, items in gemm_functions(asm).items():
        blocks, succ, _ = cfg([(label, ins) for label, ins, _ in items])
        # the inline-asm flag of each block's instructions (cfg keeps the
        # instructions in order)
        flags = [a for label, _, a in items if label is None]
        block_flags, k = [], 0
        for ins_list in blocks:
            block_flags.append(flags[k:k + len(ins_list)])
            k += len(ins_list)

        def reaches(b):
            seen, st = set(), list(succ[b])
            while st:
                x = st.pop()
                if x not in seen:
                    seen.add(x)
                    st.extend(succ[x])
            return seen
        for b, ins_list in enumerate(blocks):
            if b not in reaches(b):
                continue
            for ins, a in zip(ins_list, block_flags[b]):
                if not a and ins.startswith("s_waitcnt") and "vmcnt" in ins:
                    found.append("%s: %s" % (name, ins))
    return found


def test_loop_wait_checker_finds_a_compiler_wait():
    asm = """_Z4gemmv:
	s_mov_b32 s0, 4
.LBB0_1:
	;;#ASMSTART
	s_waitcnt vmcnt(4)
	;;#ASMEND
	s_waitcnt vmcnt(0)
	v_mov_b32_e32 v0, v1
	s_add_i32 s0, s0, -1
	s_cmp_eq_u32 s0, 0
	s_cbranch_scc0 .LBB0_1
	s_waitcnt vmcnt(0)
	s_endpgm
.Lfunc_end0:
"""
    found = compiler_waits_in_loops(asm)
    # the loop's compiler wait only: the kernel's own wait and the one after
    # the loop are not reported
    assert found == ["_Z4gemmv: s_waitcnt vmcnt(0)"], found


@pytest.mark.parametrize("src", ["dense_gemm.hip", "gemm_mx.hip"])
def test_ring_loops_hold_no_compiler_memory_waits(src, tmp_path):
    asm = compile_asm(src, str(tmp_path / (src + ".s")))
    assert gemm_functions(asm), "no GEMM kernels found in the generated code"
    found = compiler_waits_in_loops(asm)
    assert not found, "\n".join(found[:20])
