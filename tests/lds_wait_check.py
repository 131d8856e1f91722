"""Static check of the attention kernels' LDS reads on the built gfx950 code.

The mainloop issues ds_read_b128 / ds_read_b64_tr_b16 from inline assembly and
waits for them later with counted `s_waitcnt lgkmcnt(N)`.  The compiler treats
an asm output as written when the asm statement executes, so this is only
correct if no instruction reads, writes or copies a destination register of
such a read while the read is still in flight.  This module checks exactly
that on the disassembly of the shipped library:

  * LDS operations retire in issue order; `s_waitcnt lgkmcnt(N)` leaves at
    most N of them in flight (the oldest retire first).  Scalar loads and
    messages share the counter but may complete out of order, so a wait
    is assumed to retire none of them before lgkmcnt(0) and at most N LDS
    operations stay in flight whatever they do;
  * every other instruction must not name a register written by an LDS read
    that is still queued.

The scan is linear over each function's instructions (the kernels' loops
are unrolled per pipeline stage and every stage ends with its reads
retired), which only makes it stricter: state flows along the fall-through
order as well as the branches.
"""

import os
import re
import struct
import subprocess
import tempfile

LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")
_FUNC = re.compile(r"^[0-9a-f]+ <([^>]+)>:")
_LGKM = re.compile(r"lgkmcnt\((\d+)\)")


def tools_available():
    return all(os.path.exists(os.path.join(LLVM, t)) for t in ("llvm-objcopy", "llvm-objdump"))


def gfx950_code_objects(so_path):
    """The gfx950 code objects of the library's HIP fat binary (one per
    translation unit), as bytes."""
    with tempfile.TemporaryDirectory() as d:
        fat = os.path.join(d, "fat.bin")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section", f".hip_fatbin={fat}", so_path,
                        os.path.join(d, "stripped.so")], check=True, capture_output=True)
        with open(fat, "rb") as f:
            data = f.read()
    out, pos = [], 0
    while True:
        i = data.find(MAGIC, pos)
        if i < 0:
            return out
        (count,) = struct.unpack_from("<Q", data, i + len(MAGIC))
        off = i + len(MAGIC) + 8
        for _ in range(count):
            o, size, tlen = struct.unpack_from("<QQQ", data, off)
            off += 24
            triple = data[off:off + tlen].decode()
            off += tlen
            if "gfx950" in triple and size > 0:
                out.append(data[i + o:i + o + size])
        pos = i + len(MAGIC)


def disassemble(code_object):
    with tempfile.TemporaryDirectory() as d:
        p = os.path.join(d, "co.elf")
        with open(p, "wb") as f:
            f.write(code_object)
        r = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", p],
                           check=True, capture_output=True, text=True)
    return r.stdout


def functions(disasm):
    """{symbol: [instruction text, ...]} of a disassembly."""
    funcs, cur = {}, None
    for line in disasm.splitlines():
        m = _FUNC.match(line)
        if m:
            cur = funcs.setdefault(m.group(1), [])
            continue
        if cur is None or not line.startswith("\t"):
            continue
        ins = line.split("//")[0].strip()
        if ins:
            cur.append(ins)
    return funcs


def regs(operands):
    """Set of (file, index) registers named in an operand string."""
    out = set()
    for kind, lo, hi, one in _REG.findall(operands):
        if one:
            out.add((kind, int(one)))
        else:
            out.update((kind, r) for r in range(int(lo), int(hi) + 1))
    return out


def check_function(instrs):
    """Hazards in one function: (index, instruction, register, pending read)."""
    queue = []  # [(kind, dst registers, instruction text)], oldest first
    hazards = []
    for idx, ins in enumerate(instrs):
        mnem, _, ops = ins.partition(" ")
        if mnem == "s_waitcnt":
            m = _LGKM.search(ops)
            if m:
                n = int(m.group(1))
                if n == 0:
                    queue.clear()
                else:
                    # at most n operations remain; scalar loads may complete
                    # out of order, so assume they all did (the fewest LDS
                    # reads retired) and keep them until lgkmcnt(0)
                    lds = [e for e in queue if e[0] == "lds"]
                    keep = lds[len(lds) - n:] if len(lds) > n else lds
                    queue[:] = [e for e in queue if e[0] == "smem" or any(e is k for k in keep)]
            continue
        named = regs(ops)
        for _, dst, src in queue:
            hit = named & dst
            if hit:
                hazards.append((idx, ins, sorted(hit)[0], src))
        if mnem.startswith("ds_"):
            dst = set()
            if not mnem.startswith("ds_write") and "gws" not in mnem:
                # the first operand of an LDS read/permute is its destination
                first = ops.split(",")[0]
                dst = regs(first)
            queue.append(("lds", dst, ins))
        elif mnem.startswith(("s_load", "s_buffer_load", "s_sendmsg", "s_memtime", "s_memrealtime")):
            queue.append(("smem", set(), ins))
    return hazards


def attention_hazards(so_path):
    """{kernel symbol: hazards} over every attention kernel of the library;
    also returns how many asm-issued LDS reads were checked."""
    result, n_reads, n_funcs = {}, 0, 0
    for co in gfx950_code_objects(so_path):
        for name, instrs in functions(disassemble(co)).items():
            if "attn_fwd_kernel" not in name:
                continue
            n_funcs += 1
            n_reads += sum(1 for i in instrs if i.startswith(("ds_read_b128", "ds_read_b64_tr_b16")))
            h = check_function(instrs)
            if h:
                result[name] = h
    return result, n_reads, n_funcs


if __name__ == "__main__":  # manual run: python tests/lds_wait_check.py [libbsa.so]
    import sys
    so = sys.argv[1] if len(sys.argv) > 1 else os.path.join(
        os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "dynamic_block_sparse_bsa_amd", "libbsa.so")
    res, nr, nf = attention_hazards(so)
    print(f"{nf} attention kernels, {nr} LDS operand reads checked, {len(res)} with hazards")
    for k, hs in res.items():
        print(k)
        for idx, ins, reg, src in hs[:10]:
            print(f"  [{idx}] {ins}   uses {reg} of in-flight `{src}`")
