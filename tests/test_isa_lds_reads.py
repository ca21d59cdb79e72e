"""Static check of the GEMM kernels' hand-issued LDS reads (CPU only).

The GEMM core issues its fragment reads as inline ds_read_b128, whose results
arrive asynchronously; the compiler believes they are written at once.  That
is safe only while no instruction touches a read's destination registers
before an s_waitcnt lgkmcnt retires the read: a copy would read stale data,
and a register handed to something else (an address, say) would be
overwritten when the read lands.  This test compiles the library for gfx950
to assembly and walks every GEMM kernel in program order, keeping the queue
of reads in flight along every control-flow path (LDS reads retire in issue
order; lgkmcnt(N) leaves the newest N outstanding; where paths meet, their
queues are merged) and failing on any other instruction that names a
register of a read still in flight.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "grouped_expert_ffn_router_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

_REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _vregs(text):
    regs = set()
    for m in _REG.finditer(text):
        if m.group(3) is not None:
            regs.add(int(m.group(3)))
        else:
            regs.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return regs


def _kernels(asm):
    lines = asm.split("\n")
    starts = [i for i, l in enumerate(lines) if re.match(r"^_Z\w*gemm_bf16_mfma\w*:", l)]
    for s in starts:
        e = next(i for i in range(s, len(lines)) if lines[i].startswith(".Lfunc_end"))
        yield lines[s].rstrip(":"), lines[s:e]


def _instructions(body):
    """(label or None, text, in_asm) per line, comments and directives dropped."""
    out = []
    in_asm = False
    for raw in body:
        t = raw.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        m = re.match(r"^(\.LBB\w+):", t)
        if m:
            out.append((m.group(1), None, False))
            continue
        line = t.split(";")[0].strip()
        if not line or line.startswith("."):
            continue
        out.append((None, line, in_asm))
    return out


def _blocks(ins):
    """Basic blocks: list of (label, [(text, in_asm)], successor labels)."""
    blocks, cur, label = [], [], "<entry>"
    for lab, text, in_asm in ins:
        if lab is not None:
            blocks.append([label, cur])
            label, cur = lab, []
            continue
        cur.append((text, in_asm))
        if text.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            blocks.append([label, cur])
            label, cur = f"<after-{len(blocks)}>", []
    blocks.append([label, cur])
    out = []
    for k, (label, instrs) in enumerate(blocks):
        succ = []
        last = instrs[-1][0] if instrs else ""
        m = re.match(r"s_c?branch\w*\s+(\.LBB\w+)", last)
        if m:
            succ.append(m.group(1))
        if not last.startswith(("s_branch", "s_endpgm", "s_setpc")) and k + 1 < len(blocks):
            succ.append(blocks[k + 1][0])
        out.append((label, instrs, succ))
    return out


def _walk(instrs, pending, bad):
    """Advance the queue of in-flight reads through one block; record hazards."""
    pending = list(pending)
    for text, in_asm in instrs:
        m = re.match(r"s_waitcnt\b(.*)", text)
        if m:
            c = re.search(r"lgkmcnt\((\d+)\)", m.group(1))
            if c:
                keep = int(c.group(1))
                if keep < len(pending):
                    pending = pending[len(pending) - keep:]
            continue
        if in_asm and text.startswith("ds_read_b128"):
            dst = text.split()[1].rstrip(",")
            for p in pending:
                if p & _vregs(text.split(",", 1)[1]):
                    bad.append((text, "address register of a read in flight"))
            pending.append(frozenset(_vregs(dst)))
            continue
        touched = _vregs(text)
        for p in pending:
            if p & touched:
                bad.append((text, f"touches v{sorted(p)} while its LDS read is in flight"))
                break
    return pending


def _merge(a, b):
    """Queues from two paths, aligned at their newest entries; union where both have one."""
    n = max(len(a), len(b))
    a = [frozenset()] * (n - len(a)) + list(a)
    b = [frozenset()] * (n - len(b)) + list(b)
    return [x | y for x, y in zip(a, b)]


def _violations(body):
    blocks = _blocks(_instructions(body))
    index = {label: k for k, (label, _, _) in enumerate(blocks)}
    entry = {0: []}
    work = [0]
    seen = 0
    while work and seen < 20000:
        seen += 1
        k = work.pop()
        label, instrs, succ = blocks[k]
        out = _walk(instrs, entry[k], [])
        for sl in succ:
            t = index.get(sl)
            if t is None:
                continue
            new = out if t not in entry else _merge(entry[t], out)
            if t not in entry or new != entry[t]:
                entry[t] = new
                work.append(t)
    bad = []
    for k, (label, instrs, _) in enumerate(blocks):
        if k in entry:
            _walk(instrs, entry[k], bad)
    return bad


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which(HIPCC)):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "api.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "api.hip"), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-3000:]
    return out.read_text()


def test_every_gemm_kernel_leaves_in_flight_lds_reads_alone(gemm_asm):
    kernels = list(_kernels(gemm_asm))
    assert len(kernels) >= 5, "expected the five bf16 GEMM instantiations"
    for name, body in kernels:
        reads = sum(1 for l in body if l.strip().startswith("ds_read_b128"))
        assert reads > 0, f"{name}: no hand-issued LDS reads found"
        bad = _violations(body)
        assert not bad, f"{name}: {len(bad)} hazards, first: {bad[:3]}"


def test_checker_catches_planted_hazards():
    body = [";;#ASMSTART", "ds_read_b128 v[10:13], v2", ";;#ASMEND",
            "v_mov_b32_e32 v20, v11",
            ";;#ASMSTART", "s_waitcnt lgkmcnt(0)", ";;#ASMEND"]
    assert _violations(body)
    ok = [";;#ASMSTART", "ds_read_b128 v[10:13], v2", ";;#ASMEND",
          ";;#ASMSTART", "s_waitcnt lgkmcnt(0)", ";;#ASMEND", "v_mov_b32_e32 v20, v11"]
    assert not _violations(ok)
    # a read issued on the last trip of a loop and still in flight when the
    # loop exits, its register reused afterwards (the shape of a real bug
    # this check found: reads for a step past the end, then the epilogue)
    loop_exit = [".LBB0_1:", ";;#ASMSTART", "s_waitcnt lgkmcnt(0)", ";;#ASMEND",
                 "v_mfma_f32_32x32x16_bf16 a[0:15], v[10:13], v[14:17], a[0:15]",
                 ";;#ASMSTART", "ds_read_b128 v[10:13], v2", ";;#ASMEND",
                 "s_cbranch_scc1 .LBB0_1",
                 "v_or3_b32 v11, s19, v0, v244"]
    assert _violations(loop_exit)
    loop_ok = loop_exit[:-1] + [";;#ASMSTART", "s_waitcnt lgkmcnt(0)", ";;#ASMEND", "v_or3_b32 v11, s19, v0, v244"]
    assert not _violations(loop_ok)


# ------------------------------------------------ inline assembly allow-list

# The only instructions the library may issue through inline assembly: LDS
# fragment reads (whose registers the walk above tracks) and the waits and
# barrier around them.  A vector-memory load written as inline assembly is
# never allowed: the compiler treats its output register as written at once
# and may hand it to another value (an address, say) while the load is still
# in flight, which can fault the GPU.  Anything else is refused too: the
# allow-list, not a list of bad forms, decides.
ALLOWED_ASM = ("ds_read_b128", "s_waitcnt", "s_barrier")


def _asm_blocks(asm):
    """Instructions that came from inline assembly, with the function they sit in."""
    out, in_asm, fn = [], False, None
    for raw in asm.split("\n"):
        t = raw.strip()
        m = re.match(r"^(_Z\w+):", raw)
        if m:
            fn = m.group(1)
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        line = t.split(";")[0].strip()
        if in_asm and line and not line.startswith("."):
            out.append((fn, line))
    return out


def _asm_violations(asm):
    bad = []
    for fn, line in _asm_blocks(asm):
        op = line.split()[0]
        if not op.startswith(ALLOWED_ASM):
            bad.append((fn, line))
    return bad


@pytest.fixture(scope="module")
def kernels_asm(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which(HIPCC)):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa_k") / "kernels.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "kernels.hip"), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-3000:]
    return out.read_text()


def test_inline_assembly_is_only_lds_reads_waits_and_barriers(gemm_asm, kernels_asm):
    for asm in (gemm_asm, kernels_asm):
        bad = _asm_violations(asm)
        assert not bad, f"{len(bad)} inline-assembly instructions outside the allow-list, first: {bad[:3]}"
    assert _asm_blocks(gemm_asm), "the GEMM core's inline LDS reads were not found"


def test_inline_assembly_check_catches_planted_loads():
    planted = ["_Zfoo:", ";;#ASMSTART", "global_load_dwordx4 v[4:7], v[0:1], off", ";;#ASMEND"]
    assert _asm_violations("\n".join(planted))
    planted = ["_Zfoo:", ";;#ASMSTART", "buffer_load_dword v4, v0, s[0:3], 0 offen", ";;#ASMEND"]
    assert _asm_violations("\n".join(planted))
    planted = ["_Zfoo:", ";;#ASMSTART", "flat_load_dword v4, v[0:1]", ";;#ASMEND"]
    assert _asm_violations("\n".join(planted))
    ok = ["_Zfoo:", ";;#ASMSTART", "ds_read_b128 v[10:13], v2", ";;#ASMEND",
          "global_load_dwordx4 v[4:7], v[0:1], off", ";;#ASMSTART", "s_waitcnt lgkmcnt(0)", ";;#ASMEND"]
    assert not _asm_violations("\n".join(ok))


def test_sources_hold_no_other_inline_assembly():
    """Every asm statement in the library's sources is one of the allowed forms."""
    for fname in sorted(os.listdir(CSRC)):
        if not fname.endswith((".hip", ".h", ".cpp")):
            continue
        src = open(os.path.join(CSRC, fname)).read()
        for m in re.finditer(r"\basm\s+volatile\s*\(\s*\"([^\"]*)\"", src):
            op = m.group(1).split()[0]
            assert op.startswith(ALLOWED_ASM), f"{fname}: inline assembly '{m.group(1)}' outside the allow-list"
