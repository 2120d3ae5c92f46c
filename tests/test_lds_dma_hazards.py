"""Wait states around the library's global->LDS loads, checked in its own
gfx950 code (the library built from this repository, disassembled with the
ROCm LLVM tools).

The forward kernels issue their K/V/document-id loads as inline asm (a
`buffer_load ... lds` whose LDS address is M0, an asm operand the compiler
writes), and the compiler's hazard recognizer does not look inside inline
asm. Two CDNA rules apply there:
  * an LDS DMA reads M0: one wait state after a scalar write of M0;
  * a vector memory instruction reading an SGPR that a vector instruction
    wrote (readfirstlane): five wait states.
The compiler keeps both for the code it generates itself (it inserts
`s_nop` when no other instruction fills the gap), so every violation found
here comes from hand-written asm. A load that takes a stale M0 writes its
data to the previous load's LDS slot and leaves its own slot stale."""
import os
import re
import subprocess

import pytest

import block_sparse_masked_amd as lib

LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
VMEM = re.compile(r"^(buffer|global|flat|scratch)_")
LDS_DMA = re.compile(r"^(buffer_load_\w+ .*\blds\b|global_load_lds_\w+)")


def _tools():
    names = ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")
    paths = [os.path.join(LLVM, n) for n in names]
    if not all(os.access(p, os.X_OK) for p in paths):
        pytest.skip("ROCm LLVM tools not found")
    return paths


def _sregs(tok):
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m[1]), int(m[2]) + 1))
    m = re.fullmatch(r"s(\d+)", tok)
    return {int(m[1])} if m else set()


def _operands(ins):
    parts = ins.split(None, 1)
    return [t.strip() for t in parts[1].split(",")] if len(parts) > 1 else []


def _wait_states(ins):
    m = re.match(r"s_nop (\d+)", ins)
    return int(m[1]) + 1 if m else 1


def scan(kernels):
    """Violations of the two rules, per kernel: (kernel, rule, instructions)."""
    bad = []
    for name, ins in kernels.items():
        for k, i in enumerate(ins):
            if not VMEM.match(i):
                continue
            reads = set()
            for t in _operands(i)[1:]:
                reads |= _sregs(t.split()[0])
            w, j = 0, k - 1
            # walk back through straight-line code (a label or branch ends it:
            # the compiler resolves hazards across blocks for its own code)
            while j >= 0 and w < 5 and not ins[j].endswith(":"):
                q = ins[j]
                if q.startswith(("s_branch", "s_cbranch", "s_setpc", "s_endpgm")):
                    break
                ops = _operands(q)
                if LDS_DMA.match(i) and w < 1 and ops and ops[0] == "m0":
                    bad.append((name, "M0 write -> LDS DMA", ins[j:k + 1]))
                if q.startswith("v_") and ops and _sregs(ops[0]) & reads:
                    bad.append((name, "VALU SGPR write -> VMEM read", ins[j:k + 1]))
                    break
                w += _wait_states(q)
                j -= 1
    return bad


def disassemble(so_path, work):
    objcopy, bundler, objdump = _tools()
    fat = os.path.join(work, "fat.bin")
    subprocess.run([objcopy, "--dump-section", f".hip_fatbin={fat}", so_path], check=True)
    blob = open(fat, "rb").read()
    # one offload bundle per translation unit, concatenated by the linker
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), blob)]
    assert starts, "no offload bundle in the library"
    kernels = {}
    for n, s in enumerate(starts):
        e = starts[n + 1] if n + 1 < len(starts) else len(blob)
        part = os.path.join(work, f"b{n}.bin")
        co = os.path.join(work, f"b{n}.co")
        open(part, "wb").write(blob[s:e])
        subprocess.run([bundler, "--type=o", f"--targets={TARGET}", f"--input={part}",
                        f"--output={co}", "--unbundle"], check=True)
        if os.path.getsize(co) == 0:
            continue
        out = subprocess.run([objdump, "-d", "--mcpu=gfx950", co], check=True,
                             capture_output=True, text=True).stdout
        cur = None
        for line in out.splitlines():
            m = re.match(r"^[0-9a-f]+ <(.+)>:$", line)
            if m:
                cur = kernels.setdefault(m[1], [])
                continue
            if cur is None:
                continue
            text = line.split("//")[0].strip()
            if text:
                cur.append(text)
    return kernels


def test_scanner_finds_both_hazards():
    """The scanner flags a zero-wait M0 move before an LDS DMA and a
    readfirstlane into a resource word right before a buffer load, and
    accepts them once the wait states are there."""
    bad = {
        "a": ["s_mov_b32 m0, s4", "buffer_load_dwordx4 v1, s[8:11], 0 offen lds"],
        "b": ["v_readfirstlane_b32 s9, v3", "s_mov_b32 m0, s4", "s_nop 0",
              "buffer_load_dword v1, s[8:11], 0 offen lds"],
    }
    rules = sorted(r for _, r, _ in scan(bad))
    assert rules == ["M0 write -> LDS DMA", "VALU SGPR write -> VMEM read"]
    good = {
        "a": ["s_mov_b32 m0, s4", "s_nop 0", "buffer_load_dwordx4 v1, s[8:11], 0 offen lds"],
        "b": ["v_readfirstlane_b32 s9, v3", "s_nop 2", "s_mov_b32 m0, s4", "s_nop 0",
              "buffer_load_dword v1, s[8:11], 0 offen lds"],
    }
    assert scan(good) == []


M0_READERS = re.compile(r"^(s_movrel|v_movrel|s_set_gpr_idx|s_sendmsg|ds_\w*addtid|ds_gws|"
                        r"v_interp|lds_direct|lds_param)")


def m0_misuse(kernels):
    """Instructions that read M0 other than an LDS DMA. M0 is the DMA's LDS
    address, an operand of the asm that the compiler writes; no other
    instruction of the library may take M0 as an input."""
    bad = []
    for name, ins in kernels.items():
        for i in ins:
            if M0_READERS.match(i):
                bad.append((name, i))
    return bad


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    so = lib._LIB_PATH
    if not os.path.exists(so):
        pytest.skip("library not built")
    return disassemble(so, str(tmp_path_factory.mktemp("dis")))


def test_m0_read_only_by_lds_dma(kernels):
    bad = m0_misuse(kernels)
    assert not bad, bad[:8]
    fwd = [k for k in kernels if "fwd_bf16_kernel" in k]
    # every DMA still has its M0 written somewhere in the kernel
    assert all(any(_operands(i)[:1] == ["m0"] for i in kernels[k]) for k in fwd
               if any(LDS_DMA.match(i) for i in kernels[k]))


def test_library_lds_dma_wait_states(kernels):
    fwd = [k for k in kernels if "fwd_bf16_kernel" in k]
    assert fwd, "forward kernels not found in the disassembly"
    n_dma = sum(1 for k in fwd for i in kernels[k] if LDS_DMA.match(i))
    assert n_dma > 0
    bad = scan(kernels)
    msg = "\n".join(f"{n}: {r}: {' | '.join(i)}" for n, r, i in bad[:8])
    assert not bad, f"{len(bad)} wait-state violations\n{msg}"
