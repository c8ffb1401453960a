"""Wait states around the inline-assembly MFMAs (host test, no GPU).

``csrc/mfma.hpp`` issues bf16 32x32x16 MFMAs as inline assembly so that the
accumulators stay in a chosen register file. The compiler does not see the
latency of an MFMA issued that way, so the forms carry their own wait states: an
``s_nop`` before each MFMA and fences (``s_nop`` runs) after the last MFMA that
writes a set of registers. A count that is too small gives wrong results with
no error.

This test compiles the kernels that use the forms to gfx950 assembly and checks,
on every control-flow path from each inline-assembly MFMA, that the first
instruction touching its destination registers is either an MFMA accumulating
into the same registers (back-to-back accumulation needs no wait) or comes after
at least the required number of wait states. The requirement is not typed in
here: it is what the compiler's own hazard recognizer inserts between a builtin
MFMA of the same shape and an immediate consumer of its result (a VALU read, an
AGPR read, a store), calibrated on small kernels with the same flags. Each
instruction counts one wait state, ``s_nop n`` counts n + 1.
"""

import importlib.util
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "context_sparse_attention_amd", "csrc")
USERS = ["attn_token_mfma.hip", "attn_backward_mfma.hip"]
MFMA = "v_mfma_f32_32x32x16_bf16"

CALIBRATION = r"""
#include <hip/hip_runtime.h>
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
// result read by the vector ALU right away
__global__ void cal_valu(const bf16x8* a, float* out) {
  f32x16 c = {};
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[threadIdx.x], a[threadIdx.x + 64], c, 0, 0, 0);
  out[threadIdx.x] = c[0] * 3.0f;
}
// result stored right away
__global__ void cal_store(const bf16x8* a, f32x16* out) {
  f32x16 c = {};
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[threadIdx.x], a[threadIdx.x + 64], c, 0, 0, 0);
  out[threadIdx.x] = c;
}
// result fed to a dependent MFMA as an A operand (after a conversion)
__global__ void cal_chain(const bf16x8* a, f32x16* out) {
  f32x16 c = {};
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[threadIdx.x], a[threadIdx.x + 64], c, 0, 0, 0);
  bf16x8 p;
  for (int j = 0; j < 8; ++j) p[j] = (__bf16)c[j];
  f32x16 d = {};
  d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p, a[threadIdx.x], d, 0, 0, 0);
  out[threadIdx.x] = d;
}
"""


def _flags():
    spec = importlib.util.spec_from_file_location(
        "csa_build", os.path.join(ROOT, "context_sparse_attention_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    flags = [f for f in mod.FLAGS if f not in ("-fPIC",)]
    return mod.HIPCC, flags


def _assemble(src_path, out_path):
    hipcc, flags = _flags()
    cmd = [hipcc, *flags, "--cuda-device-only", "-S", src_path, "-o", out_path]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out_path).read()


_REG_RANGE = re.compile(r"\b([va])\[(\d+):(\d+)\]")
_REG_ONE = re.compile(r"\b([va])(\d+)\b")


def _regs(operands):
    out = set()
    for f, a, b in _REG_RANGE.findall(operands):
        out.update((f, r) for r in range(int(a), int(b) + 1))
    stripped = _REG_RANGE.sub(" ", operands)
    for f, a in _REG_ONE.findall(stripped):
        out.add((f, int(a)))
    return out


class Instr:
    def __init__(self, text, in_asm):
        parts = text.split(None, 1)
        self.op = parts[0]
        self.operands = parts[1] if len(parts) > 1 else ""
        self.in_asm = in_asm
        ops = [o.strip() for o in self.operands.split(",")]
        self.regs = _regs(self.operands)
        self.dst = _regs(ops[0]) if ops and ops[0] else set()
        self.srcc = _regs(ops[3]) if self.op == MFMA and len(ops) > 3 else set()

    def waits(self):
        if self.op == "s_nop":
            return int(self.operands.split()[0], 0) + 1
        return 1


def _functions(asm):
    """name -> (instructions, label -> index)."""
    funcs = {}
    lines = asm.splitlines()
    i = 0
    while i < len(lines):
        m = re.match(r"^([A-Za-z_][\w.$]*):\s*(;.*)?$", lines[i])
        if m and not m.group(1).startswith(".L"):
            name = m.group(1)
            ins, labels, in_asm = [], {}, False
            i += 1
            while i < len(lines) and not lines[i].startswith(".Lfunc_end"):
                raw = lines[i].strip()
                i += 1
                if raw.startswith(";;#ASMSTART"):
                    in_asm = True
                    continue
                if raw.startswith(";;#ASMEND"):
                    in_asm = False
                    continue
                lm = re.match(r"^(\.?L\w+|\w+):", raw)
                if lm:
                    labels[lm.group(1)] = len(ins)
                    continue
                if not raw or raw.startswith(";") or raw.startswith("."):
                    continue
                ins.append(Instr(raw.split(";")[0].strip(), in_asm))
            funcs[name] = (ins, labels)
        i += 1
    return funcs


def _succ(ins, labels, j):
    op = ins[j].op
    if op == "s_endpgm":
        return []
    if op == "s_branch":
        return [labels[ins[j].operands.split()[0]]]
    if op.startswith("s_cbranch"):
        return [labels[ins[j].operands.split()[0]], j + 1]
    return [j + 1] if j + 1 < len(ins) else []


def _first_uses(ins, labels, i, limit):
    """(index, wait states before it, is_chain) of the first access to MFMA i's
    destination on each path, exploring until `limit` wait states have passed."""
    dst = ins[i].dst
    found, seen = [], set()
    stack = [(s, 0) for s in _succ(ins, labels, i)]
    while stack:
        j, w = stack.pop()
        if (j, w) in seen or j >= len(ins):
            continue
        seen.add((j, w))
        x = ins[j]
        if x.regs & dst:
            chain = x.op == MFMA and x.dst == dst and x.srcc == dst
            found.append((j, w, chain))
            continue
        w2 = w + x.waits()
        if w2 >= limit:
            continue
        stack.extend((s, w2) for s in _succ(ins, labels, j))
    return found


@pytest.fixture(scope="module")
def asm_dir():
    with tempfile.TemporaryDirectory(prefix="csa_hazard_") as d:
        yield d


_CACHE = {}


def _kernel_funcs(src, asm_dir):
    if src not in _CACHE:
        _CACHE[src] = _functions(_assemble(os.path.join(CSRC, src),
                                           os.path.join(asm_dir, src + ".s")))
    return _CACHE[src]


@pytest.fixture(scope="module")
def requirement(asm_dir):
    """Wait states the compiler places between a builtin 32x32x16 MFMA and an
    immediate consumer of its result (the largest over the calibration kernels)."""
    src = os.path.join(asm_dir, "cal.hip")
    with open(src, "w") as f:
        f.write(CALIBRATION)
    funcs = _functions(_assemble(src, os.path.join(asm_dir, "cal.s")))
    req = {}
    for name, (ins, labels) in funcs.items():
        kind = re.search(r"cal_(\w+?)P", name)
        if not kind:
            continue
        first = next(k for k, x in enumerate(ins) if x.op == MFMA)
        uses = _first_uses(ins, labels, first, 10_000)
        assert uses, name
        req[kind.group(1)] = min(w for _, w, chain in uses if not chain)
    assert set(req) == {"valu", "store", "chain"}, req
    return req


def test_calibration_is_plausible(requirement):
    # the compiler must demand some wait after a 32x32x16 result, and the fences
    # of mfma.hpp (16 and 24 wait states) must cover it
    worst = max(requirement.values())
    assert 4 <= worst <= 16, requirement


@pytest.mark.parametrize("src", USERS)
def test_inline_mfma_results_are_waited_for(src, asm_dir, requirement):
    need = max(requirement.values())
    funcs = _kernel_funcs(src, asm_dir)
    checked, problems = 0, []
    for name, (ins, labels) in funcs.items():
        for i, x in enumerate(ins):
            if not (x.in_asm and x.op == MFMA):
                continue
            checked += 1
            for j, w, chain in _first_uses(ins, labels, i, need):
                if not chain and w < need:
                    problems.append(f"{name[:60]}: MFMA #{i} -> {ins[j].op} #{j} after {w} "
                                    f"wait states (< {need})")
    print(f"{src}: {checked} inline-assembly MFMAs checked against {need} wait states "
          f"(calibration {requirement})")
    assert checked > 0, f"{src}: no inline-assembly MFMA found"
    assert not problems, "\n".join(problems[:10])


@pytest.fixture(scope="module")
def operand_requirement(asm_dir):
    """Wait states the compiler places between a VALU write of an MFMA's A operand
    and the MFMA (the conversion in the calibration's chained kernel)."""
    src = os.path.join(asm_dir, "cal_ops.hip")
    with open(src, "w") as f:
        f.write(CALIBRATION)
    funcs = _functions(_assemble(src, os.path.join(asm_dir, "cal_ops.s")))
    name = next(n for n in funcs if "cal_chain" in n)
    ins, _ = funcs[name]
    second = [k for k, x in enumerate(ins) if x.op == MFMA][1]
    a_regs = _regs(ins[second].operands.split(",")[1])
    w = 0
    for k in range(second - 1, -1, -1):
        if ins[k].op.startswith("v_") and ins[k].dst & a_regs:
            return w
        w += ins[k].waits()
    raise AssertionError("no VALU writer of the second MFMA's A operand")


@pytest.mark.parametrize("src", USERS)
def test_inline_mfma_operands_are_ready(src, asm_dir, operand_requirement):
    """Every inline-assembly MFMA is preceded, inside its own asm block, by an
    s_nop covering what a VALU write of an operand right before it (which the
    compiler may schedule there) needs."""
    funcs = _kernel_funcs(src, asm_dir)
    for name, (ins, labels) in funcs.items():
        for i, x in enumerate(ins):
            if x.in_asm and x.op == MFMA:
                prev = ins[i - 1]
                assert prev.in_asm and prev.op == "s_nop" and \
                    prev.waits() >= max(1, operand_requirement), \
                    f"{name[:60]}: MFMA #{i} lacks its leading s_nop"


SYNTHETIC = """
kern:
;;#ASMSTART
\ts_nop 1
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]
;;#ASMEND
.LBB0_1:
;;#ASMSTART
\ts_nop 1
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[8:11], v[4:7], a[0:15]
;;#ASMEND
\tv_add_u32_e32 v20, 1, v20
\ts_cbranch_scc1 .LBB0_1
\ts_nop {n}
\tv_accvgpr_read_b32 v30, a3
\ts_endpgm
.Lfunc_end0:
"""


@pytest.mark.parametrize("n", [2, 7])
def test_checker_flags_a_short_wait(n):
    """The path checker itself: after the loop, an AGPR read n + 1 + 2 wait states
    past the last MFMA; the loop's back edge leads to an accumulation (fine)."""
    ins, labels = _functions(SYNTHETIC.format(n=n))["kern"]
    mf = [i for i, x in enumerate(ins) if x.op == MFMA]
    assert len(mf) == 2
    uses = _first_uses(ins, labels, mf[1], 100)
    chains = [w for _, w, c in uses if c]
    reads = [w for j, w, c in uses if not c]
    assert chains and reads == [2 + n + 1]   # v_add, s_cbranch, then s_nop n
    assert min(reads) < 16
