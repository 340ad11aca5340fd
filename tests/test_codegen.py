"""Checks on the gfx950 code the pipelined kernels compile to (CPU only: hipcc
cross-compiles, nothing runs).

The pipelined SpMM kernels issue their global loads from inline assembly and
wait for them with explicit `s_waitcnt vmcnt` statements that take the
destination registers as operands.  The data of such a load arrives
asynchronously, so no instruction may read or overwrite its destination
registers until a wait has retired it -- otherwise a register copy would read
stale data, or a register reused for an address would be overwritten by the
late load.  Vector-memory operations retire in issue order, and
`s_waitcnt vmcnt(N)` returns once at most the N newest are outstanding; the
checker models exactly that, counting the compiler's own memory operations
too, and replays every loop body once with the state its back edge carries.

The direct global->LDS loads are preceded by a write of M0 in the same inline
assembly.  M0 is a register the compiler reserves for itself, so the second
check requires that no instruction outside those assembly blocks reads or
writes M0 in any kernel built with them.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_matmul_ffns_amd", "csrc")

VMEM_PREFIXES = ("global_", "buffer_", "scratch_", "flat_")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def _regs(text):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]", text):
        out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"\bv(\d+)\b", text):
        out.add(int(m.group(1)))
    return out


def _split(s):
    parts = s.split(None, 1)
    ops = parts[1] if len(parts) > 1 else ""
    return parts[0], [o.strip() for o in ops.split(",")] if ops else []


def _code(line):
    return line.split(";")[0].strip()


def _blocks(asm_lines):
    """Basic blocks of a kernel body: list of (label or None, [(line no, text, in_asm)], successors)."""
    items, in_asm = [], False
    for i, line in enumerate(asm_lines):
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        c = _code(s)
        if not c or c.startswith("."):
            if re.match(r"^\.?[A-Za-z_][\w.$]*:$", c):
                items.append(("label", i, c[:-1], in_asm))
            continue
        items.append(("insn", i, c, in_asm))
    blocks, cur = [], None
    for kind, i, c, in_asm in items:
        if kind == "label":
            cur = {"label": c, "insns": [], "succ": []}
            blocks.append(cur)
            continue
        if cur is None:
            cur = {"label": None, "insns": [], "succ": []}
            blocks.append(cur)
        cur["insns"].append((i, c, in_asm))
        mnem = c.split()[0]
        if mnem == "s_branch" or mnem.startswith("s_cbranch") or mnem in ("s_endpgm", "s_setpc_b64"):
            cur["end"] = mnem
            cur = {"label": None, "insns": [], "succ": []}
            blocks.append(cur)
    index = {b["label"]: k for k, b in enumerate(blocks) if b["label"]}
    for k, b in enumerate(blocks):
        end = b.get("end")
        if end in ("s_endpgm", "s_setpc_b64"):
            continue
        if end:
            ops = b["insns"][-1][1].split(None, 1)
            target = ops[1].strip() if len(ops) > 1 else ""
            if target in index:
                b["succ"].append(index[target])
            if end == "s_branch":
                continue
        if k + 1 < len(blocks):
            b["succ"].append(k + 1)
    return blocks


def async_register_violations(asm_lines):
    """Instructions that touch the destination of an inline-asm load before a wait retires it.

    Returns sorted (line number, instruction) pairs.  Every vector-memory instruction (inline
    assembly or compiler-issued) joins an in-order queue of at most 63 (the counter's range);
    `s_waitcnt vmcnt(N)` keeps only the N newest; the destination registers of inline-assembly
    loads still queued are pending.  The queue states are propagated over the control-flow
    graph until no block sees a new one."""
    blocks = _blocks(asm_lines)
    bad = set()
    seen = set()
    # state: (queue, EXEC known to hold every lane, SGPR pairs known to hold a full-EXEC copy)
    work = [(0, (), True, frozenset())] if blocks else []
    while work:
        k, queue, full, saved = work.pop()
        if (k, queue, full, saved) in seen:
            continue
        seen.add((k, queue, full, saved))
        q = list(queue)
        for i, c, in_asm in blocks[k]["insns"]:
            mnem, ops = _split(c)
            if not in_asm:
                full, saved = _exec_step(mnem, ops, full, saved)
            if mnem == "s_waitcnt":
                m = re.search(r"vmcnt\((\d+)\)", c)
                if m:
                    n = int(m.group(1))
                    q = q[len(q) - n:] if n else []
                continue
            pending = set().union(*[e[1] for e in q]) if q else set()
            vmem = mnem.startswith(VMEM_PREFIXES)
            is_load = vmem and "load" in mnem and "lds" not in mnem
            sources = ops[1:] if is_load else ops
            if _regs(",".join(sources)) & pending:
                bad.add((i + 1, c))
            if is_load and in_asm and ops:
                dest = frozenset(_regs(ops[0]))
                if dest & pending:
                    bad.add((i + 1, c))
                q.append((None, dest))
            elif vmem:
                if is_load and ops and _regs(ops[0]) & pending:
                    bad.add((i + 1, c))
                q.append((None, frozenset()))
            elif ops and _regs(ops[0]) & pending:
                bad.add((i + 1, c))
            # at most 63 outstanding; entries older than the oldest inline-asm load can never
            # make a register pending, and compiler entries differ only in their position
            q = [(None, e[1]) for e in q[-63:]]
            while q and not q[0][1]:
                q.pop(0)
        succ = blocks[k]["succ"]
        end = blocks[k].get("end")
        if full and end in ("s_cbranch_execz", "s_cbranch_execnz") and len(succ) == 2:
            # with every lane active, execz never branches and execnz always does
            succ = [succ[1]] if end == "s_cbranch_execz" else [succ[0]]
        for s in succ:
            work.append((s, tuple(q), full, saved))
    return sorted(bad)


def _exec_step(mnem, ops, full, saved):
    """Track whether EXEC holds every lane (kernels start with whole waves) through the compiler's
    save / mask / restore idioms; anything else that writes EXEC makes it unknown."""
    dst = ops[0] if ops else ""
    if mnem in ("s_and_saveexec_b64", "s_andn2_saveexec_b64", "s_or_saveexec_b64", "s_xor_saveexec_b64"):
        saved = (saved | {dst}) if full else (saved - {dst})
        return (full and mnem == "s_or_saveexec_b64"), saved
    if mnem == "s_mov_b64" and len(ops) == 2 and ops[1] == "exec":
        return full, (saved | {dst}) if full else (saved - {dst})
    if dst == "exec":
        if mnem == "s_mov_b64":
            return ops[1] in saved or ops[1] == "-1", saved
        if mnem == "s_or_b64" and "exec" in ops[1:]:
            other = [o for o in ops[1:] if o != "exec"]
            return full or bool(other and other[0] in saved), saved
        return False, saved
    if mnem.startswith("v_cmpx"):
        return False, saved
    if dst.startswith("s") and saved:
        saved = frozenset(r for r in saved if r != dst)
    return full, saved


def m0_violations(asm_lines):
    """Instructions outside inline assembly that name M0."""
    bad, in_asm = [], False
    for i, line in enumerate(asm_lines):
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not s or s.startswith((";", ".")) or s.endswith(":"):
            continue
        if re.search(r"\bm0\b", s.split(";")[0]) and not in_asm:
            bad.append((i + 1, s))
    return bad


def _kernels(asm_text, prefix):
    """Device kernel bodies (entry label .. the function's end label) whose symbol starts with prefix."""
    out, cur, body = {}, None, []
    for line in asm_text.splitlines():
        label = line.split(";")[0].strip()
        if label.startswith(prefix) and label.endswith(":"):
            cur, body = label[:-1], []
            continue
        if cur is not None:
            if label.startswith(".Lfunc_end"):
                out[cur] = body
                cur = None
                continue
            body.append(line)
    return out


def _compile(tmp_path, src):
    from sparse_matmul_ffns_amd import build
    asm = tmp_path / (os.path.splitext(src)[0] + ".s")
    cmd = [_hipcc(), *build.FLAGS, "--cuda-device-only", "-S", "-o", str(asm), os.path.join(CSRC, src)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return asm.read_text()


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.parametrize("src,prefix,load,min_kernels", [
    ("spmm_dma.hip", "_ZN3nms15spmm_dma_kernel", "global_load_dwordx4", 3),
    ("spmm_vnm.hip", "_ZN3nms19spmm_vnm_reg_kernel", "buffer_load_dword", 1),
])
def test_pipelined_spmm_never_touches_in_flight_registers(tmp_path, src, prefix, load, min_kernels):
    kernels = _kernels(_compile(tmp_path, src), prefix)
    assert len(kernels) >= min_kernels
    for name, lines in kernels.items():
        assert any(load in l for l in lines), name
        bad = async_register_violations(lines)
        assert not bad, f"{name}: {bad[:5]}"


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.parametrize("src", ["spmm_dma.hip", "spmm_vnm.hip", "spmm_nt.hip", "spmm_w4.hip", "sddmm.hip", "lowrank.hip"])
def test_m0_written_only_by_the_direct_load_helpers(tmp_path, src):
    kernels = _kernels(_compile(tmp_path, src), "_ZN3nms")
    assert kernels
    for name, lines in kernels.items():
        bad = m0_violations(lines)
        assert not bad, f"{name}: {bad[:5]}"


def test_checker_catches_a_reused_register():
    # a load whose destination is overwritten before the wait must be flagged
    asm = """
    ;;#ASMSTART
    global_load_dwordx4 v[4:7], v[0:1], off
    ;;#ASMEND
    v_add_u32_e32 v5, 1, v9
    ;;#ASMSTART
    s_waitcnt vmcnt(0)
    ;;#ASMEND
    v_mov_b32_e32 v4, v10
    """.splitlines()
    bad = async_register_violations(asm)
    assert len(bad) == 1 and "v5" in bad[0][1]


def test_checker_keeps_the_newest_loads_pending():
    # vmcnt(1) retires the older load only; the newer one's register stays pending
    asm = """
    ;;#ASMSTART
    buffer_load_dword v1, v0, s[4:7], 0 offen
    ;;#ASMEND
    ;;#ASMSTART
    buffer_load_dword v2, v0, s[4:7], 0 offen
    ;;#ASMEND
    ;;#ASMSTART
    s_waitcnt vmcnt(1)
    ;;#ASMEND
    v_mov_b32_e32 v3, v1
    v_mov_b32_e32 v3, v2
    """.splitlines()
    bad = async_register_violations(asm)
    assert len(bad) == 1 and "v2" in bad[0][1]


def test_checker_follows_a_loop_back_edge():
    # the load issued at the end of the body is still pending at the top of the next iteration
    asm = """
    .LBB0_1:
    v_add_u32_e32 v7, v2, v3
    ;;#ASMSTART
    buffer_load_dword v2, v0, s[4:7], 0 offen
    ;;#ASMEND
    s_cbranch_scc1 .LBB0_1
    ;;#ASMSTART
    s_waitcnt vmcnt(0)
    ;;#ASMEND
    """.splitlines()
    bad = async_register_violations(asm)
    assert bad and "v2" in bad[0][1]


def test_checker_counts_compiler_memory_operations():
    # a compiler store issued after the load makes vmcnt(1) retire the load
    asm = """
    ;;#ASMSTART
    buffer_load_dword v1, v0, s[4:7], 0 offen
    ;;#ASMEND
    global_store_dword v[8:9], v5, off
    s_waitcnt vmcnt(1)
    v_mov_b32_e32 v3, v1
    """.splitlines()
    assert async_register_violations(asm) == []


def test_m0_checker_flags_a_compiler_write():
    asm = """
    ;;#ASMSTART
    s_mov_b32 m0, s4
    global_load_lds_dwordx4 v0, off
    ;;#ASMEND
    s_mov_b32 m0, -1
    """.splitlines()
    bad = m0_violations(asm)
    assert len(bad) == 1 and "-1" in bad[0][1]


def test_checker_resolves_uniform_exec_branches():
    # with every lane active, the fallthrough of execnz (back into the loop) is never taken, but
    # after a divergent mask it may be
    loop = """
    .LBB0_1:
    v_add_u32_e32 v7, v2, v3
    ;;#ASMSTART
    buffer_load_dword v2, v0, s[4:7], 0 offen
    ;;#ASMEND
    s_cbranch_execnz .LBB0_2
    s_branch .LBB0_1
    .LBB0_2:
    ;;#ASMSTART
    s_waitcnt vmcnt(0)
    ;;#ASMEND
    s_endpgm
    """
    assert async_register_violations(loop.splitlines()) == []
    divergent = "v_cmp_gt_u32_e32 vcc, 8, v1\n    s_and_saveexec_b64 s[8:9], vcc\n" + loop
    bad = async_register_violations(divergent.splitlines())
    assert bad and "v2" in bad[0][1]


def test_n8_sorting_network_sorts_every_input():
    """The 8-input comparator network of the one-pass N:8 prune (csrc/prune.hip) sorts descending.
    By the 0-1 principle a comparator network sorts every input iff it sorts all 2^8 inputs of
    zeros and ones, so the 256 cases decide it."""
    src = open(os.path.join(CSRC, "prune.hip")).read()
    i = src.index("8-input sorting network of 19 comparators")
    block = src[i:src.index("thr = srt[N - 1]", i)]
    pairs = [(int(a), int(b)) for a, b in re.findall(r"cx\((\d+), (\d+)\)", block)]
    assert len(pairs) == 19
    for bits in range(256):
        v = [(bits >> p) & 1 for p in range(8)]
        for a, b in pairs:
            hi, lo = max(v[a], v[b]), min(v[a], v[b])
            v[a], v[b] = hi, lo
        assert v == sorted(v, reverse=True), (bits, v)
