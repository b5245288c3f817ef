"""Static checks of the accumulation chains in libbitgemm's own GEMM kernels,
read from the AMDGCN the library's sources compile to (hipcc --cuda-device-only -S).

The order fields of a descriptor fix, for every output, one chain of matrix
instructions over ascending k; a schedule field (tile, waves, stages, walk,
load path) may change which lane owns which output but not that chain
("Taming Bitwise Behavior", section 6: static checking that a variant leaves
the reduction tree unchanged).  What the ISA of each compiled variant can show
without evaluating addresses:

  * every matrix instruction is the one the variant's template names;
  * every one accumulates in place (its C operand is its destination), so no
    chain is split into partial accumulators that a later add would combine;
  * inside each loop that runs the k walk, no other instruction writes an
    accumulator (no scaling, no partial sums, no register shuffles);
  * in each such loop every accumulator receives the same number of matrix
    instructions, a multiple of the k-steps one turn holds, and there are as
    many accumulators as the wave owns output blocks.

The k order itself (which k block each instruction reads) comes from LDS
addresses and is checked at run time, bit for bit against the oracle."""
import hashlib
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fixed_order_fp_amd", "csrc")
CACHE = os.path.join(ROOT, "fixed_order_fp_amd", "_build", "isa")

MFMA = {0: "v_mfma_f32_32x32x16_bf16", 1: "v_mfma_f32_16x16x32_bf16",
        2: "v_mfma_i32_32x32x32_i8", 3: "v_mfma_i32_16x16x64_i8"}
INSTR_K = {0: 16, 1: 32, 2: 32, 3: 64}
BLOCK = {0: 32, 1: 16, 2: 32, 3: 16}  # output block edge of the instruction

STORES = ("ds_write", "ds_store", "global_store", "buffer_store", "scratch_store", "flat_store",
          "global_load_lds", "buffer_load_dword lds", "global_atomic", "buffer_atomic", "ds_add", "s_")


def device_asm(src):
    """AMDGCN text of one source file, compiled as the library is (cached by
    the source's and its headers' contents)."""
    sys.path.insert(0, ROOT)
    from fixed_order_fp_amd import build as B
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    with open(os.path.join(ROOT, "include", "bitgemm.h"), "rb") as fh:
        h.update(fh.read())
    os.makedirs(CACHE, exist_ok=True)
    out = os.path.join(CACHE, f"{os.path.splitext(src)[0]}.{h.hexdigest()[:16]}.s")
    if not os.path.exists(out):
        flags = [f for f in B.FLAGS if f != "-fPIC"]
        cmd = [B.HIPCC, *flags, f"-DBG_PROFILE_HASH=0x{B.profile_hash():016x}ull", "--cuda-device-only", "-S",
               os.path.join(CSRC, src), "-o", out + ".tmp"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed:\n{r.stderr}")
        os.replace(out + ".tmp", out)
    with open(out) as f:
        return f.read()


def kernels(asm):
    """{mangled name: [instruction lines]} for every kernel in the text."""
    out = {}
    name, body = None, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            name, body = m.group(1), []
            out[name] = body
            continue
        if name is None:
            continue
        if line.startswith(".Lfunc_end"):
            name = None
            continue
        body.append(line)
    return out


def template_ints(mangled):
    """Integer and bool template arguments, in order ("Li320E" -> 320, "Lb1E" -> 1)."""
    m = re.search(r"I((?:L[ib]\d+E)+)E", mangled)
    return [int(x) for x in re.findall(r"L[ib](\d+)E", m.group(1))] if m else []


REG = re.compile(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b")


def regs(operand):
    m = REG.search(operand)
    if not m:
        return None
    if m.group(1):
        return (m.group(1), int(m.group(2)), int(m.group(3)))
    return (m.group(4), int(m.group(5)), int(m.group(5)))


def overlaps(a, b):
    return a[0] == b[0] and a[1] <= b[2] and b[1] <= a[2]


def instructions(lines):
    """(index, mnemonic, operands) of the instruction lines."""
    out = []
    for i, line in enumerate(lines):
        s = line.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        parts = s.split(None, 1)
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        out.append((i, parts[0], ops))
    return out


def loops(lines):
    """{loop header: [line indices]} of the loops, from the loop annotations
    LLVM writes beside each basic block's label (a rotated loop may place
    blocks of its body before the header)."""
    out = {}
    cur = None
    label = re.compile(r"^(\.LBB\d+_\d+|; %bb\.\d+):")
    for i, line in enumerate(lines):
        m = label.match(line)
        if m:
            cur = None
            # the annotation is on the label line or on the comment lines after it
            j = i
            while j < len(lines) and (j == i or lines[j].lstrip().startswith(";")):
                a = re.search(r"in Loop: Header=(BB\d+_\d+) Depth=(\d+)", lines[j])
                h = re.search(r"Loop Header: Depth=(\d+)", lines[j])
                if a:
                    cur = a.group(1)
                    break
                if h and m.group(1).startswith(".LBB"):
                    cur = m.group(1)[2:]
                    break
                j += 1
        if cur is not None:
            out.setdefault(cur, []).append(i)
    return out


def check_kernel(lines, instr, ksteps, blocks):
    """Problems found in one kernel (an empty list certifies it)."""
    problems = []
    ins = instructions(lines)
    mf = [(i, op, ops) for i, op, ops in ins if op.startswith("v_mfma")]
    for i, op, ops in mf:
        if op != MFMA[instr]:
            problems.append(f"line {i}: {op}, expected {MFMA[instr]}")
        if len(ops) != 4 or regs(ops[0]) != regs(ops[3]):
            problems.append(f"line {i}: {op} does not accumulate in place ({', '.join(ops)})")
    n_walk = 0
    for head, idx in loops(lines).items():
        keep = set(idx)
        body = [(i, op, ops) for i, op, ops in ins if i in keep]
        a = head
        accs = {}
        for i, op, ops in body:
            if op.startswith("v_mfma"):
                r = regs(ops[0])
                accs[r] = accs.get(r, 0) + 1
        if not accs:
            continue  # not a k walk
        n_walk += 1
        counts = set(accs.values())
        if len(counts) != 1:
            problems.append(f"loop at {a}: accumulators get different numbers of instructions {sorted(counts)}")
        elif next(iter(counts)) % ksteps:
            problems.append(f"loop at {a}: {next(iter(counts))} instructions per accumulator, not a multiple "
                            f"of {ksteps} k-steps")
        if len(accs) != blocks:
            problems.append(f"loop at {a}: {len(accs)} accumulators, the wave owns {blocks} blocks")
        for i, op, ops in body:
            if op.startswith("v_mfma") or op.startswith(STORES) or not ops:
                continue
            d = regs(ops[0])
            if d and any(overlaps(d, r) for r in accs):
                problems.append(f"line {i}: {op} writes accumulator register {ops[0]} inside the k walk")
    if mf and n_walk == 0:
        problems.append("no loop holds the matrix instructions")
    return problems


def gemm_variants(asm):
    """(name, instr, k-steps per turn, blocks per wave) of every bf16 GEMM kernel."""
    out = []
    for name, lines in kernels(asm).items():
        t = template_ints(name)
        if "gemm_bf16_pipe_kernel" in name:          # <BM, BN, WM, WN, NS, OUT, RED>
            bm, bn, wm, wn = t[0], t[1], t[2], t[3]
            out.append((name, lines, 0, 32 // INSTR_K[0], (bm // wm // 32) * (bn // wn // 32)))
        elif "gemm_bf16_direct_kernel" in name:      # <INSTR, BM, BN, WM, WN, OUT_BF16, PARTIAL>, BK 64
            i, bm, bn, wm, wn = t[0], t[1], t[2], t[3], t[4]
            e = BLOCK[i]
            out.append((name, lines, i, 64 // INSTR_K[i], (bm // wm // e) * (bn // wn // e)))
        elif "gemm_bf16_kernel" in name:             # <INSTR, BM, BN, BK, WM, WN, OUT_BF16, PARTIAL>
            i, bm, bn, bk, wm, wn = t[0], t[1], t[2], t[3], t[4], t[5]
            e = BLOCK[i]
            out.append((name, lines, i, bk // INSTR_K[i], (bm // wm // e) * (bn // wn // e)))
    return out


def w8a8_variants(asm):
    out = []
    for name, lines in kernels(asm).items():
        t = template_ints(name)
        if "w8a8_pipe_kernel" in name:               # <BM, BN, WM, WN, NS, MODE>, k tiles of 64 bytes
            bm, bn, wm, wn = t[0], t[1], t[2], t[3]
            out.append((name, lines, 2, 64 // INSTR_K[2], (bm // wm // 32) * (bn // wn // 32)))
        elif "w8a8_kernel" in name:                  # <INSTR, BM, BN, WM, WN, ACC_OUT>, k tiles of 128 bytes
            i, bm, bn, wm, wn = t[0], t[1], t[2], t[3], t[4]
            e = BLOCK[i]
            out.append((name, lines, i, 128 // INSTR_K[i], (bm // wm // e) * (bn // wn // e)))
    return out
