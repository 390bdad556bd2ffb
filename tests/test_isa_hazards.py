"""Wait-state checks on the compiled gfx950 device code (no GPU needed).

The matrix-core kernels issue some MFMAs as inline asm (to pin accumulators
to VGPRs or AGPRs).  The compiler pads the MFMAs it emits itself against
data hazards but does not look inside asm, so those MFMAs carry their NOPs by
hand.  The hardware does not interlock these cases; a missing wait state
reads a stale register and gives silently wrong scores.  This test compiles
the library's device code to assembly and walks each MFMA's neighbourhood in
program order:

  * a VALU instruction writing a VGPR that an MFMA reads (A, B or C operand)
    must be at least 2 wait states before it;
  * a VALU or memory instruction reading or writing an MFMA's destination
    must be at least 11 wait states after it (an 8-pass 32x32 XDL op).

Wait states are counted as one per instruction, N + 1 per `s_nop N`.  The
walk is linear (it does not follow branches): a regression guard for the
straight-line loop bodies, not a proof.

The direct global->LDS loads are inline asm that write M0 (the LDS base).
The compiler is told M0 is clobbered, but M0 is a register it may also
allocate; in a kernel whose asm writes M0, no instruction the compiler
emits may read or write M0, or a value it keeps there would be overwritten.
"""

import os
import re
import shutil
import subprocess

import pytest

from sequence_sharded_mla_amd import build as B

VALU_TO_MFMA = 2
MFMA_TO_USE = 11

_REG = re.compile(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out.update((m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1))
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _instructions(asm):
    """Per kernel: list of (mnemonic, operand text) in program order; labels
    and directives are dropped."""
    kernels, cur = {}, None
    for raw in asm.split("\n"):
        line = raw.split(";")[0].strip()
        if not line:
            continue
        if line.endswith(":") and not line.startswith("."):
            name = line[:-1]
            if name.startswith("_Z"):
                cur = kernels.setdefault(name, [])
            continue
        if cur is None or line.startswith("."):
            continue
        parts = line.split(None, 1)
        cur.append((parts[0], parts[1] if len(parts) > 1 else ""))
    return kernels


_M0 = re.compile(r"\bm0\b")


def _m0_uses(asm):
    """Per kernel: (number of inline-asm lines naming m0, compiler-emitted
    instructions naming m0)."""
    out, cur, inasm = {}, None, False
    for raw in asm.split("\n"):
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            inasm = True
            continue
        if s.startswith(";;#ASMEND"):
            inasm = False
            continue
        line = s.split(";")[0].strip()
        if not line:
            continue
        if line.endswith(":") and line.startswith("_Z"):
            cur = out.setdefault(line[:-1], [0, []])
            continue
        if cur is None or line.startswith(".") or not _M0.search(line):
            continue
        if inasm:
            cur[0] += 1
        else:
            cur[1].append(line)
    return out


def _m0_conflicts(uses):
    return [f"{k}: compiler-emitted '{ins[0]}' in a kernel whose asm writes m0"
            for k, (n_asm, ins) in uses.items() if n_asm and ins]


def _wait_states(mn, ops):
    return int(ops.split()[0], 0) + 1 if mn == "s_nop" else 1


def _dst_src(mn, ops):
    fields = [f.strip() for f in ops.split(",")]
    if mn.startswith(("global_store", "buffer_store", "ds_write", "ds_store", "flat_store")):
        return set(), _regs(ops)
    if not fields:
        return set(), set()
    return _regs(fields[0]), _regs(",".join(fields[1:]))


def _check(kernel, ins):
    problems = []
    for i, (mn, ops) in enumerate(ins):
        if not mn.startswith("v_mfma"):
            continue
        fields = [f.strip() for f in ops.split(",")]
        srcs = _regs(",".join(fields[1:4]))
        dst = _regs(fields[0])
        ws, j = 0, i - 1
        while j >= 0 and ws < VALU_TO_MFMA:
            pm, po = ins[j]
            if pm.startswith("v_") and not pm.startswith("v_mfma"):
                d, _ = _dst_src(pm, po)
                if d & srcs:
                    problems.append(f"{kernel}: '{pm} {po}' then '{mn} {ops}' after {ws} wait states")
                    break
            ws += _wait_states(pm, po)
            j -= 1
        ws, j = 0, i + 1
        while j < len(ins) and ws < MFMA_TO_USE:
            nm, no = ins[j]
            if nm.startswith("v_mfma"):
                nf = [f.strip() for f in no.split(",")]
                # chained accumulation into the same registers is forwarded
                if _regs(nf[0]) == dst and _regs(nf[3]) == dst:
                    ws += 1
                    j += 1
                    continue
                if _regs(",".join(nf[1:3])) & dst:
                    problems.append(f"{kernel}: '{mn} {ops}' result read as A/B by '{nm} {no}'")
                break
            if nm.startswith(("v_", "global_", "buffer_", "ds_", "flat_")):
                d, s = _dst_src(nm, no)
                if (d | s) & dst:
                    problems.append(f"{kernel}: '{mn} {ops}' then '{nm} {no}' after {ws} wait states")
                    break
            ws += _wait_states(nm, no)
            j += 1
    return problems


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    if not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "api.s"
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [B.HIPCC] + flags + ["-S", "--cuda-device-only", "-o", str(out), B.SOURCES[0]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


def test_mfma_kernels_present(device_asm):
    kernels = _instructions(device_asm)
    names = [k for k, ins in kernels.items() if any(m.startswith("v_mfma") for m, _ in ins)]
    assert any("decode_mfma_bf16_kernel" in k for k in names)
    assert sum("decode_mfma_fp8_kernel" in k for k in names) >= 2


def test_mfma_wait_states(device_asm):
    problems = []
    for kernel, ins in _instructions(device_asm).items():
        problems += _check(kernel, ins)
    assert not problems, "\n".join(problems[:20])


def test_checker_catches_a_missing_wait_state():
    """The walk itself flags a VALU write right before an MFMA read, and a
    VALU read right after an MFMA write."""
    bad = [("v_cvt_scalef32_pk_bf16_fp8", "v13, v20, 1.0"),
           ("v_mfma_f32_32x32x16_bf16", "v[18:33], v[10:13], v[70:73], v[18:33]"),
           ("s_nop", "7"),
           ("v_add_f32", "v40, v18, v41")]
    probs = _check("k", bad)
    assert len(probs) == 2
    good = [("v_cvt_scalef32_pk_bf16_fp8", "v13, v20, 1.0"),
            ("s_nop", "2"),
            ("v_mfma_f32_32x32x16_bf16", "v[18:33], v[10:13], v[70:73], v[18:33]"),
            ("s_nop", "7"), ("s_nop", "7"),
            ("v_add_f32", "v40, v18, v41")]
    assert _check("k", good) == []


def test_m0_left_to_the_asm(device_asm):
    uses = _m0_uses(device_asm)
    writers = [k for k, (n, _) in uses.items() if n and ("decode_mfma" in k)]
    assert len(writers) >= 3, "the decode kernels' direct-to-LDS loads were expected to set m0 in asm"
    problems = _m0_conflicts(uses)
    assert not problems, "\n".join(problems[:20])


def test_m0_checker_flags_a_compiler_use():
    asm = "\n".join([
        "_Zk:",
        ";;#ASMSTART",
        "s_mov_b32 m0, s4",
        "global_load_lds_dwordx4 v1, s[2:3]",
        ";;#ASMEND",
        "v_writelane_b32 v5, s6, m0",
        "_Zq:",
        "s_mov_b32 m0, s7",
    ])
    uses = _m0_uses(asm)
    assert uses["_Zk"][0] == 1 and len(uses["_Zk"][1]) == 1
    assert len(_m0_conflicts(uses)) == 1   # _Zq uses m0 only in compiler code: no asm writer
