"""Checks of the built gfx950 code object of libog.so (the library's own
device code, extracted from the shared library, one code object per
compiled unit):

- the DPP read hazard: a register read through DPP (the source of a
  v_*_dpp instruction) is never written by a VALU instruction fewer than two
  wait states before the read.  The compiler does not model this hazard
  through inline asm, so the library's asm blocks start with s_nop 1; the
  disassembly confirms it;
- no kernel spills registers to scratch memory or keeps any other data
  there (a kernel that does is correct but many times slower: a lambda the
  compiler did not inline once put a kernel's argument block in scratch
  and made its buffer descriptors non-uniform); the code-object metadata
  records both."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "fp32_blocked_gemm_amd", "libog.so")
LLVM = "/opt/rocm/llvm/bin"


def _code_objects(d):
    """The gfx950 code objects of libog.so: its .hip_fatbin section holds one
    offload bundle per compiled unit, each unbundled on its own."""
    bundler = os.path.join(LLVM, "clang-offload-bundler")
    fat = os.path.join(d, "fat.bin")
    # objcopy writes its output over its input when no output file is named:
    # work on a copy, so the library that this process has loaded is never
    # rewritten under it
    lib, scrap = os.path.join(d, "lib.so"), os.path.join(d, "scrap.so")
    shutil.copyfile(LIB, lib)
    subprocess.run(["objcopy", "--dump-section", f".hip_fatbin={fat}", lib, scrap], check=True)
    with open(fat, "rb") as f:
        blob = f.read()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    starts = [m.start() for m in re.finditer(re.escape(magic), blob)]
    assert starts and starts[0] == 0, "no offload bundle in .hip_fatbin"
    cos = []
    for i, (a, b) in enumerate(zip(starts, starts[1:] + [len(blob)])):
        part, co = os.path.join(d, f"part{i}.bin"), os.path.join(d, f"dev{i}.co")
        with open(part, "wb") as f:
            f.write(blob[a:b])
        subprocess.run([bundler, "--unbundle", "--type=o",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={part}",
                        f"--output={co}"], check=True)
        cos.append(co)
    return cos


def _notes(d):
    return "".join(subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", co], check=True,
                                  capture_output=True, text=True).stdout for co in _code_objects(d))


def _tools_or_skip():
    for tool in ("clang-offload-bundler", "llvm-objdump", "llvm-readelf"):
        if not os.path.exists(os.path.join(LLVM, tool)):
            pytest.skip(f"{tool} is missing")
    if not (os.path.exists(LIB) and shutil.which("objcopy")):
        pytest.skip("libog.so or objcopy is missing")


def test_no_kernel_spills():
    _tools_or_skip()
    with tempfile.TemporaryDirectory() as d:
        notes = _notes(d)
    names = re.findall(r"^\s*\.name:\s+(\S+)", notes, flags=re.M)
    spills = [int(v) for v in re.findall(r"\.vgpr_spill_count:\s+(\d+)", notes)]
    sspills = [int(v) for v in re.findall(r"\.sgpr_spill_count:\s+(\d+)", notes)]
    assert spills and len(spills) == len(sspills)
    bad = [n for n, v, s in zip(names, spills, sspills) if v or s]
    assert not bad, f"kernels spilling registers: {bad[:5]}"
    private = [int(v) for v in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", notes)]
    assert len(private) == len(names)
    bad = [n for n, v in zip(names, private) if v]
    assert not bad, f"kernels using scratch memory: {bad[:5]}"


def test_every_host_kernel_has_device_code():
    """Each kernel the host code can launch (its mangled name registered in
    the library) is in the gfx950 code object.  A library whose host and
    device passes saw different sources would launch a kernel that does not
    exist, which the HIP runtime turns into an abort."""
    _tools_or_skip()
    with tempfile.TemporaryDirectory() as d:
        notes = _notes(d)
    device = set(re.findall(r"^\s*\.name:\s+(\S+)", notes, flags=re.M))
    with open(LIB, "rb") as f:
        blob = f.read()
    host = {m.decode() for m in re.findall(rb"_ZN2og\d+[a-z_]+kernelI[0-9A-Za-z_]*?EEvNS_7ProblemE",
                                            blob)}
    host = {n for n in host if "__device_stub__" not in n}  # the host-side launch stubs
    assert host, "no kernel names found in the library"
    missing = sorted(host - device)
    assert not missing, f"{len(missing)} kernels registered on the host have no device code: {missing[:3]}"


def _disassemble():
    _tools_or_skip()
    with tempfile.TemporaryDirectory() as d:
        out = "".join(subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", co],
                                     check=True, capture_output=True, text=True).stdout
                      for co in _code_objects(d))
    return out


def _regs(tok):
    """VGPR numbers named by an operand token: v5 or v[4:7]."""
    m = re.fullmatch(r"v(\d+)", tok)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def _hazards(text):
    insts = []
    for line in text.splitlines():
        s = line.split("//")[0].strip()
        if not s or s.endswith(":") or s.startswith((".", ";")):
            continue
        insts.append(s)
    bad = []
    for i, s in enumerate(insts):
        m = re.match(r"(v_\w+_dpp)\s+(\S+),\s*(\S+)", s)
        if not m:
            continue
        src = _regs(m.group(3).rstrip(","))
        waits = 0
        j = i - 1
        while j >= 0 and waits < 2:
            p = insts[j]
            if p.startswith("s_nop"):
                waits += int(p.split()[1], 0) + 1 if len(p.split()) > 1 else 1
            else:
                pm = re.match(r"(v_\w+)\s+([^,\s]+)", p)
                if (pm and not pm.group(1).startswith(("v_cmp", "v_readfirstlane", "v_readlane"))
                        and _regs(pm.group(2)) & src):
                    bad.append(f"{p}  ->  {s}")
                    break
                waits += 1
            j -= 1
    return bad


def test_no_dpp_read_after_valu_write():
    text = _disassemble()
    assert "_dpp" in text, "the library's DPP kernels were not found in the disassembly"
    bad = _hazards(text)
    assert not bad, f"{len(bad)} DPP hazards, e.g. {bad[:3]}"


def test_the_scan_finds_a_planted_hazard():
    """The scanner itself flags a DPP read right after a VALU write."""
    text = ("\tv_mov_b32_e32 v7, v1\n"
            "\tv_fmac_f32_dpp v2, v7, v3 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
            "\tv_mov_b32_e32 v9, v1\n\ts_nop 1\n"
            "\tv_fmac_f32_dpp v2, v9, v3 row_newbcast:1 row_mask:0xf bank_mask:0xf\n")
    assert len(_hazards(text)) == 1


def _waterfalls(text):
    """Kernels with a buffer access inside a waterfall loop: the descriptor
    was in vector registers, so the compiler loops over its distinct values
    (s_and_saveexec, the access, s_xor exec, s_cbranch_execnz)."""
    kernel, insts, found = None, [], set()
    for line in text.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
        if m:
            kernel, insts = m.group(1), []
            continue
        s = line.split("//")[0].strip()
        if not s or s.endswith(":") or s.startswith((".", ";")):
            continue
        insts.append(s)
        if s.startswith("s_cbranch_execnz") and len(insts) >= 4:
            w = insts[-4:-1]
            if (w[-1].startswith("s_xor_b64 exec, exec") and
                    any(x.startswith("buffer_") for x in w[:-1]) and
                    any(x.startswith("s_and_saveexec") for x in insts[-6:-2])):
                found.add(kernel)
    return sorted(found)


def test_no_buffer_access_in_a_waterfall_loop():
    """Every staging load's descriptor is wave-uniform and held in scalar
    registers.  A descriptor the compiler believes divergent is read through
    a waterfall loop, which slowed the 4096^3 product's main loop by 8 %
    (a 64-bit channel index in the store epilogue once caused it)."""
    text = _disassemble()
    bad = _waterfalls(text)
    assert not bad, f"{len(bad)} kernels with waterfall buffer accesses, e.g. {bad[:3]}"


def test_the_scan_finds_a_planted_waterfall():
    text = ("0000000000001000 <k>:\n"
            "\tv_readfirstlane_b32 s8, v2\n\tv_cmp_eq_u64_e64 s[2:3], s[8:9], v[2:3]\n"
            "\ts_and_saveexec_b64 s[2:3], s[2:3]\n"
            "\tbuffer_load_dwordx4 v[130:133], v7, s[8:11], 0 offen\n"
            "\ts_xor_b64 exec, exec, s[2:3]\n\ts_cbranch_execnz 65521\n")
    assert _waterfalls(text) == ["k"]
