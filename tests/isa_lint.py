"""Reads the gfx950 machine code of the built library (this repository's own build) and lists the
places where one MFMA takes another MFMA's result as its accumulator (SrcC).

The compiler schedules an accumulator read of the immediately preceding MFMA's result with no
independent instructions between them whenever the registers coincide exactly, whatever the two
instructions' shapes. Chains of one MFMA instruction are correct that way; a chain that mixed the
16x16x32 and 16x16x16 f16 products gave wrong values in the product placed second. The lint finds
every accumulator dependency whose producer is an MFMA of another instruction, so a test can require
that there are none.
"""
import os
import re
import subprocess

LLVM = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin")
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

_REG = re.compile(r"^([va])(?:\[(\d+):(\d+)\]|(\d+))$")


def regs(op):
    """The register numbers an operand names ('v7', 'v[4:7]', 'a[0:3]'), or [] for anything else."""
    m = _REG.match(op.strip())
    if not m:
        return []
    kind = m.group(1)
    if m.group(4) is not None:
        return [(kind, int(m.group(4)))]
    return [(kind, r) for r in range(int(m.group(2)), int(m.group(3)) + 1)]


def disassemble(lib_path, workdir):
    """Disassembly text of every gfx950 code object in the library's offload section, one per
    translation unit."""
    sec = os.path.join(workdir, "fatbin.bin")
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section", ".hip_fatbin=" + sec, lib_path,
                    os.path.join(workdir, "host.o")], check=True, capture_output=True)
    data = open(sec, "rb").read()
    starts = []
    i = data.find(MAGIC)
    while i >= 0:
        starts.append(i)
        i = data.find(MAGIC, i + 1)
    out = []
    for n, s in enumerate(starts):
        e = starts[n + 1] if n + 1 < len(starts) else len(data)
        b = os.path.join(workdir, "bundle%d.bin" % n)
        co = os.path.join(workdir, "bundle%d.co" % n)
        open(b, "wb").write(data[s:e])
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                        "--targets=" + TARGET, "--input=" + b, "--output=" + co], check=True, capture_output=True)
        out.append(subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", co],
                                  check=True, capture_output=True, text=True).stdout)
    return out


def functions(text):
    """{symbol: [(mnemonic, [operands])]} from llvm-objdump output."""
    funcs, cur = {}, None
    for line in text.splitlines():
        h = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
        if h:
            cur = funcs.setdefault(h.group(1), [])
            continue
        if cur is None or not line.startswith("\t") and not line.startswith(" "):
            continue
        body = line.split("//")[0].strip()
        if not body:
            continue
        parts = body.split(None, 1)
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        cur.append((parts[0], ops))
    return funcs


def _writes(mn, ops):
    """Registers an instruction writes (first operand, both for swaps); stores and scalar,
    branch and wait instructions write none."""
    if mn.startswith(("s_", "global_store", "buffer_store", "flat_store", "scratch_store", "ds_write",
                      "ds_store", "exp")) or not ops:
        return []
    if "_swap" in mn and mn.startswith("v_"):
        return regs(ops[0]) + regs(ops[1])
    return regs(ops[0])


def mixed_accumulator_chains(insts, window=64):
    """Every MFMA whose SrcC was last written by an MFMA of another instruction, as tuples
    (reader index, reader, writer, wait states between them). The body is walked twice so that a
    dependency carried around a loop is seen too; wait states count instructions between the two and
    the idle states of s_nop."""
    n = len(insts)
    last = {}  # register -> (index in the doubled walk, mnemonic, wait states so far)
    ws = 0
    found = []
    for k in range(2 * n):
        mn, ops = insts[k % n]
        if mn.startswith("v_mfma") and len(ops) >= 4:
            src_c = regs(ops[3])
            if src_c:
                prods = {last.get(r) for r in src_c}
                for p in prods:
                    if p is None or not p[1].startswith("v_mfma"):
                        continue
                    if p[1] != mn and ws - p[2] < window:
                        found.append((k % n, mn, p[1], ws - p[2]))
        w = 1
        if mn == "s_nop" and ops:
            w = int(ops[0], 0) + 1
        ws += w
        for r in _writes(mn, ops):
            last[r] = (k, mn, ws)
    return sorted(set(found))
