"""The LDS DMA loads are inline assembly, which the compiler's hazard
recognizer does not look into, so each load carries its own wait states
(load_lds16<W>): s_nop 4 by default, s_nop 0 only in steady-state main loops
whose descriptors come from scalar arithmetic. This test reads the gfx950
code objects of the built libmoe.so and checks, for every buffer_load ... lds,
the two rules the compiler would otherwise enforce:

* no VALU write of an SGPR the load reads (its descriptor) within the 5 wait
  states before it (v_readfirstlane, v_readlane restoring a spilled SGPR,
  v_cmp_*_e64 or carry-out SGPR destinations);
* M0 is not written by the instruction immediately before it (1 wait state).

A load within 5 wait states of a branch target has a second path in; those
must not occur either. Runs on the CPU (llvm-objdump on the shipped binary).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "routing_grouped_gemm_softmax_amd", "libmoe.so")
LLVM = "/opt/rocm/llvm/bin"
TOOLS = ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")


def _disassemble(tmp_path):
    fb = tmp_path / "fatbin.bin"
    # An explicit output file: with the input alone, llvm-objcopy rewrites
    # the library in place.
    subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fb}", LIB, str(tmp_path / "lib_copy.so")],
                   check=True)
    data = fb.read_bytes()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    starts = [m.start() for m in re.finditer(re.escape(magic), data)]
    texts = []
    for n, a in enumerate(starts):
        b = starts[n + 1] if n + 1 < len(starts) else len(data)
        bundle, co = tmp_path / f"b{n}", tmp_path / f"co{n}.o"
        bundle.write_bytes(data[a:b])
        subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o", f"--input={bundle}",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"], check=True)
        texts.append(subprocess.run([f"{LLVM}/llvm-objdump", "-d", "--mcpu=gfx950", str(co)], check=True,
                                    capture_output=True, text=True).stdout)
    return texts


_SREG = re.compile(r"\bs\[(\d+):(\d+)\]|\bs(\d+)\b")


def _sregs(op):
    out = set()
    for m in _SREG.finditer(op):
        if m.group(1):
            out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
        else:
            out.add(int(m.group(3)))
    return out


def _valu_sgpr_dst(mn, ops):
    if not mn.startswith("v_"):
        return set()
    if mn.startswith(("v_readfirstlane", "v_readlane")) or (mn.startswith("v_cmp") and mn.endswith("_e64")):
        return _sregs(ops[0]) if ops else set()
    if "_co_" in mn or mn.startswith("v_div_scale"):
        return _sregs(ops[1]) if len(ops) > 1 else set()
    return set()


def _scan(text):
    issues, n_dma = [], 0
    for func in re.split(r"\n(?=[0-9a-f]+ <)", text):
        hdr = func.split("\n", 1)[0]
        m = re.match(r"([0-9a-f]+) <", hdr)
        base = int(m.group(1), 16) if m else None
        lines = []
        for ln in func.split("\n")[1:]:
            m = re.match(r"\s+(\S+)\s*([^/]*?)\s*//\s*([0-9A-F]+):", ln)
            if m:
                ops = [o.strip() for o in m.group(2).split(",")] if m.group(2) else []
                lines.append((m.group(1), ops, int(m.group(3), 16), ln))
        targets = set()
        for mn, _, _, ln in lines:
            t = re.search(r"<[^>+]*\+0x([0-9a-f]+)>", ln)
            if (mn.startswith("s_cbranch") or mn == "s_branch") and t:
                targets.add(int(t.group(1), 16))
        for i, (mn, ops, addr, ln) in enumerate(lines):
            if not (mn.startswith("buffer_load") and ln.split("//")[0].rstrip().endswith(" lds")):
                continue
            n_dma += 1
            reads = _sregs(ops[1]) if len(ops) > 1 else set()
            if i and lines[i - 1][0].startswith("s_") and lines[i - 1][1][:1] == ["m0"]:
                issues.append(f"{hdr} {addr:#x}: M0 written just before")
            ws, j = 0, i - 1
            while j >= 0 and ws < 5:
                jmn, jops, jaddr, _ = lines[j]
                if _valu_sgpr_dst(jmn, jops) & reads:
                    issues.append(f"{hdr} {addr:#x}: {jmn} {','.join(jops)} {ws} wait states before")
                    break
                ws += int(jops[0], 0) + 1 if jmn == "s_nop" else 1
                if base is not None and jaddr - base in targets and ws < 5:
                    issues.append(f"{hdr} {addr:#x}: branch target {ws} wait states before")
                    break
                j -= 1
    return issues, n_dma


def test_lds_dma_loads_carry_their_wait_states(tmp_path):
    if not os.path.exists(LIB):
        pytest.skip("libmoe.so is not built")
    if not all(shutil.which(t) or os.path.exists(f"{LLVM}/{t}") for t in TOOLS):
        pytest.skip("ROCm llvm tools not found")
    issues, total = [], 0
    for text in _disassemble(tmp_path):
        iss, n = _scan(text)
        issues += iss
        total += n
    assert total > 0, "no LDS DMA loads found: the scan no longer matches the disassembly"
    assert not issues, "\n".join(issues[:20])


def test_scan_catches_an_unguarded_load():
    """The scanner itself flags the two hazards on a hand-written listing."""
    listing = """0000000000001000 <k>:
	v_readfirstlane_b32 s42, v133                              // 000000001000: 7E540585
	buffer_load_dwordx4 v58, s[40:43], 0 offen lds             // 000000001004: E05D1000 800A003A
	s_mov_b32 m0, s29                                          // 00000000100C: BEFC001D
	buffer_load_dwordx4 v60, s[44:47], 0 offen lds             // 000000001010: E05D1000 800B003C
	s_nop 4                                                    // 000000001018: BF800004
	buffer_load_dwordx4 v61, s[40:43], 0 offen lds             // 00000000101C: E05D1000 800A003D
"""
    issues, n = _scan(listing)
    assert n == 3
    assert len(issues) == 2 and "v_readfirstlane" in issues[0] and "M0" in issues[1]
