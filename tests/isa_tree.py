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
addresses and is checked at run time, bit for bit against the oracle.

Canonical dependence-tree signatures (further below) read the tree of one
output back from the code of the split-K combine (the partials' loads
resolved to their plane index, then the adds) and of the row reduction (the
leaf's loads numbered by offset, the fold, the DPP steps and the readlanes),
so that variants and builds can be compared with each other and with the
tree the definition gives."""
import hashlib
import os
from fractions import Fraction
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


def device_asm(src, opt="-O3"):
    """AMDGCN text of one source file, compiled as the library is (cached by
    the source's and its headers' contents); `opt` replaces the optimisation
    level, for a second build to compare with the library's."""
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
    out = os.path.join(CACHE, f"{os.path.splitext(src)[0]}.{opt.lstrip('-')}.{h.hexdigest()[:16]}.s")
    if not os.path.exists(out):
        flags = [opt if f == "-O3" else f for f in B.FLAGS if f != "-fPIC"]
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
    """Problems found in one kernel (an empty list certifies it).  `blocks`
    is the number of output blocks a wave owns, or a set of them for a kernel
    that runs two tile shapes (each must have its own k walk)."""
    problems = []
    allowed = set(blocks) if isinstance(blocks, (set, frozenset)) else {blocks}
    seen = set()
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
        seen.add(len(accs))
        if len(accs) not in allowed:
            problems.append(f"loop at {a}: {len(accs)} accumulators, the wave owns {sorted(allowed)} blocks")
        for i, op, ops in body:
            if op.startswith("v_mfma") or op.startswith(STORES) or not ops:
                continue
            d = regs(ops[0])
            if d and any(overlaps(d, r) for r in accs):
                problems.append(f"line {i}: {op} writes accumulator register {ops[0]} inside the k walk")
    if mf and n_walk == 0:
        problems.append("no loop holds the matrix instructions")
    if mf and n_walk and not allowed <= seen:
        problems.append(f"no k walk for the tiles whose waves own {sorted(allowed - seen)} blocks")
    return problems


def gemm_variants(asm):
    """(name, instr, k-steps per turn, blocks per wave) of every bf16 GEMM kernel."""
    out = []
    for name, lines in kernels(asm).items():
        t = template_ints(name)
        if "gemm_bf16_pipe_kernel" in name:          # <BM, BN, WM, WN, NS, OUT, RED, BK>
            if t[5] == 4:  # the two-chain free-order twin: no single-chain contract
                continue
            bm, bn, wm, wn, bk = t[0], t[1], t[2], t[3], t[7]
            out.append((name, lines, 0, bk // INSTR_K[0], (bm // wm // 32) * (bn // wn // 32)))
        elif "gemm_bf16_pipe_dual_kernel" in name:   # <BM, BN, WM, WN, NS, BM2, BN2, WM2, WN2, NS2, OUT, BK>
            b1 = (t[0] // t[2] // 32) * (t[1] // t[3] // 32)
            b2 = (t[5] // t[7] // 32) * (t[6] // t[8] // 32)
            out.append((name, lines, 0, t[11] // INSTR_K[0], {b1, b2}))
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
        if "w8a8_pipe_kernel" in name:               # <BM, BN, WM, WN, NS, MODE>: k tiles of 64 bytes, 128 at NS 2
            bm, bn, wm, wn, ns = t[0], t[1], t[2], t[3], t[4]
            pk = 128 if ns <= 3 else 64  # two or three stages: 128-byte k tiles
            out.append((name, lines, 2, pk // INSTR_K[2], (bm // wm // 32) * (bn // wn // 32)))
        elif "w8a8_kernel" in name:                  # <INSTR, BM, BN, WM, WN, ACC_OUT>, k tiles of 128 bytes
            i, bm, bn, wm, wn = t[0], t[1], t[2], t[3], t[4]
            e = BLOCK[i]
            out.append((name, lines, i, 128 // INSTR_K[i], (bm // wm // e) * (bn // wn // e)))
    return out


# ---------------------------------------------------------------------------
# Canonical dependence-tree signatures ("Taming Bitwise Behavior", section 6:
# the reduction tree read back from the compiled code, so that two variants
# or two builds can be compared; Table 3 lists an AMDGCN checker).  Each
# signature is a string that names the floating-point operations of one
# output's reduction and how they nest, with the registers renamed away:
# equal strings mean the same tree, whatever the schedule or the build.
# fp32 addition is commutative bit for bit on non-NaN operands, so the two
# operands of an add are put in a canonical order; association is kept.
# ---------------------------------------------------------------------------
def balanced_tree(leaves):
    """The balanced tree over `leaves` (strings), neighbours first, an odd
    last node carried up, written as nested sums with commutative operands
    sorted -- built from the definition, independently of any kernel."""
    nodes = list(leaves)
    while len(nodes) > 1:
        nxt = [canon_add(nodes[i], nodes[i + 1]) for i in range(0, len(nodes) - 1, 2)]
        if len(nodes) % 2:
            nxt.append(nodes[-1])
        nodes = nxt
    return nodes[0]


def canon_add(a, b):
    return "(" + " + ".join(sorted((a, b))) + ")"


def gemm_chain_signature(lines, instr, k_per_turn):
    """The tree of one GEMM output inside one split, as the ISA shows it: a
    single chain of the descriptor's matrix instruction accumulating in place,
    one instruction per instruction_k of k.  Returns None when the kernel
    does not have that shape (check_kernel then names the problem)."""
    ins = instructions(lines)
    accs = {}
    for head, idx in loops(lines).items():
        keep = set(idx)
        for i, op, ops in ins:
            if i in keep and op.startswith("v_mfma"):
                if len(ops) != 4 or regs(ops[0]) != regs(ops[3]):
                    return None
                accs.setdefault(head, {}).setdefault(regs(ops[0]), []).append(op)
    if not accs:
        return None
    shapes = set()
    for head, per in accs.items():
        for r, ops in per.items():
            if len(set(ops)) != 1:
                return None
            shapes.add((ops[0], len(ops)))
    if len({s[0] for s in shapes}) != 1:
        return None
    mnem = next(iter(shapes))[0]
    # per turn of k_per_turn, one instruction per instruction_k
    per_turn = {n for _, n in shapes}
    if per_turn != {k_per_turn // INSTR_K[instr]}:
        return None
    return f"chain[{mnem}, in place, k step {INSTR_K[instr]}, ascending]"


def _pair(op):
    m = re.match(r"s\[(\d+):(\d+)\]$", op)
    return (int(m.group(1)), int(m.group(2))) if m else None


def _sym_loads(ins):
    """Plane index of each dword load of a split-K combine kernel: partial s
    sits at base + s * plane elements, the base being (idx << 2) + the
    workspace pointer and the plane count a scalar pair, the offset formed as
    (plane << shift), as a 64-bit multiply by a constant (low half from the
    pair's low register) or as a shifted scalar pair.  Returns {instruction
    index: (loaded register, plane)} or None when an address is not of that form or two
    loads use different plane counts."""
    val = {}      # low VGPR of an address pair -> (plane multiple, plane pair)
    sval = {}     # scalar pair -> (plane multiple, plane pair)
    loads = {}
    planes = set()
    for i, op, ops in ins:
        if op == "s_lshl_b64" and len(ops) == 3 and _pair(ops[0]) and _pair(ops[1]) and ops[2].isdigit():
            sval[_pair(ops[0])] = (Fraction(2 ** int(ops[2]), 4), _pair(ops[1]))
        elif op == "v_lshl_add_u64" and len(ops) == 4:
            d, a, sh, b = ops
            dr = regs(d)
            if a.startswith("v[") and _pair(b) and sh == "2" and regs(a)[1] not in val:
                val[dr[1]] = (Fraction(0), None)                      # (idx << 2) + workspace
            elif _pair(a) and b.startswith("v[") and regs(b)[1] in val and sh.isdigit():
                k, q = val[regs(b)[1]]
                val[dr[1]] = (k + Fraction(2 ** int(sh), 4), _pair(a))
                planes.add(_pair(a))
            elif a.startswith("v[") and regs(a)[1] in val and sh == "0" and _pair(b) in sval:
                k, q = val[regs(a)[1]]
                k2, q2 = sval[_pair(b)]
                val[dr[1]] = (k + k2, q2)
                planes.add(q2)
            else:
                val.pop(dr[1], None)
        elif op == "v_mad_u64_u32" and len(ops) == 5:
            d, _, a, c, b = ops
            dr = regs(d)
            if re.match(r"s\d+$", a) and any(int(a[1:]) == q[1] for q in planes):
                pass                                                  # the high half of a product below
            elif re.match(r"s\d+$", a) and c.isdigit() and b.startswith("v[") and regs(b)[1] in val:
                k, q = val[regs(b)[1]]
                lo = int(a[1:])
                val[dr[1]] = (k + Fraction(int(c), 4), (lo, lo + 1))   # low half: base + c * plane
                planes.add((lo, lo + 1))
            else:
                val.pop(dr[1], None)
        elif op == "global_load_dword" and len(ops) >= 2:
            r = regs(ops[1])
            if r is None or r[1] not in val or val[r[1]][0].denominator != 1:
                return None
            loads[i] = (regs(ops[0])[1], int(val[r[1]][0]))
    if len(planes) > 1:
        return None
    return loads


def combine_tree_signature(lines):
    """The tree a split-K combine kernel applies to the partials P0..P(S-1)
    of one output, read from its adds, and the planes it loads (None if it
    cannot be read).  Any other instruction writing a register that held a
    partial sum passes it on as an opaque function of it (the rounding to
    bf16 is integer code), so the stored value shows the sum it came from;
    a register it writes from nothing tracked is dropped."""
    ins = instructions(lines)
    loads = _sym_loads(ins)
    if not loads:
        return None
    expr = {}
    last = None
    for i, op, ops in ins:
        if i in loads:
            r, plane = loads[i]
            expr[r] = f"P{plane}"
        elif op.startswith("v_add_f32") and len(ops) == 3:
            a, b = regs(ops[1]), regs(ops[2])
            d = regs(ops[0])[1]
            if a is None or b is None or a[1] not in expr or b[1] not in expr:
                expr.pop(d, None)
                continue
            expr[d] = canon_add(expr[a[1]].split("cvt:")[-1], expr[b[1]].split("cvt:")[-1])
        elif op.startswith(("global_store_dword", "global_store_short")):
            r = regs(ops[1])
            if r is not None and r[1] in expr:
                last = expr[r[1]].split("cvt:")[-1]
        elif op.startswith("v_") and ops and regs(ops[0]) and regs(ops[0])[0] == "v":
            d = regs(ops[0])
            srcs = [expr[regs(o)[1]] for o in ops[1:] if regs(o) and regs(o)[0] == "v" and regs(o)[1] in expr]
            for k in range(d[1], d[2] + 1):
                if srcs and k == d[1]:
                    expr[k] = "cvt:" + max(srcs, key=len)
                else:
                    expr.pop(k, None)
    return last, sorted(p for _, p in loads.values())


def leaf_chain(n, fused=True):
    """The leaf fold of n elements e0.. in index order with no seed, from
    the definition: (sum, sum of squares) as canonical expression strings."""
    sm = "e0"
    sq = "(e0*e0)"
    for i in range(1, n):
        sm = canon_add(sm, f"e{i}")
        sq = f"fma(e{i},e{i},{sq})" if fused else canon_add(sq, f"(e{i}*e{i})")
    return sm, sq


def wave_tree(x):
    """The count-up wave tree over one value per lane, from the definition:
    DPP row shifts 1, 2, 4, 8 (each lane at the end of a run of 2d lanes adds
    the run's left half), then the four row roots as (r0 + r1) + (r2 + r3)."""
    t = x
    for d in (1, 2, 4, 8):
        t = f"S{d}({t})"
    return canon_add(canon_add(f"L15[{t}]", f"L31[{t}]"), canon_add(f"L47[{t}]", f"L63[{t}]"))


def _src(expr, o):
    r = regs(o)
    if r is not None and r[0] == "v":
        return expr.get(("v", r[1]))
    m = re.match(r"s(\d+)$", o)
    if m:
        return expr.get(("s", int(m.group(1))))
    return None


def row_tree_signature(lines, bf16):
    """The row reduction's tree for one row block, read from the kernel's
    whole-leaf path: the straight-line code from the first vector load of
    the leaf through the readlanes that finish the wave tree.  Loaded dwords
    are numbered from the leaf's start (offset / 4), a bf16 pair unpacked by
    the shift and the mask becomes elements 2n and 2n + 1, and adds, fused
    multiply-adds, multiplies, DPP-shifted adds with their lane selects and
    readlanes build expressions.  Returns the expressions of the two wave
    roots (sum, sum of squares), or None."""
    ins = instructions(lines)
    k0 = next((k for k, (i, op, ops) in enumerate(ins) if op == "global_load_dwordx4"), None)
    if k0 is None:
        return None
    expr = {}
    roots = []
    for i, op, ops in ins[k0:]:
        if op == "global_load_dwordx4":
            d = regs(ops[0])
            m = re.search(r"offset:(\d+)", " ".join(ops))
            base = (int(m.group(1)) if m else 0) // 4
            for j in range(4):
                expr[("v", d[1] + j)] = ("w", base + j)
            continue
        if op.startswith(("s_waitcnt", "s_nop", "v_cmp", "s_cmp")) or op.startswith("s_and_b64"):
            continue
        if op.startswith(("s_barrier", "ds_write", "ds_store", "s_cbranch", "s_branch", "global_store")):
            break
        d = regs(ops[0]) if ops else None
        if op == "v_lshlrev_b32_e32" and ops[1] == "16":
            w = _src(expr, ops[2])
            val = f"e{2 * w[1]}" if isinstance(w, tuple) and bf16 else None
        elif op == "v_and_b32_e32" and ops[1].lower() == "0xffff0000":
            w = _src(expr, ops[2])
            val = f"e{2 * w[1] + 1}" if isinstance(w, tuple) and bf16 else None
        elif op.startswith("v_add_f32_dpp"):
            sh = re.search(r"row_shr:(\d+)", ",".join(ops))
            a = _src(expr, ops[1])
            val = ("dpp", int(sh.group(1)) if sh else 0, a)
        elif op.startswith("v_cndmask_b32"):
            x, y = _src(expr, ops[1]), _src(expr, ops[2])
            val = None
            for new, old in ((x, y), (y, x)):
                if isinstance(new, tuple) and new[0] == "dpp" and new[2] == old:
                    val = f"S{new[1]}({old})"
        elif op == "v_readlane_b32":
            m = re.match(r"s(\d+)$", ops[0])
            v = _src(expr, ops[1])
            if m:
                expr[("s", int(m.group(1)))] = f"L{ops[2]}[{v}]" if isinstance(v, str) else None
            continue
        elif op.startswith(("v_mov_b32", "v_mov_b32_e32")):
            val = _src(expr, ops[1])
        elif op.startswith("v_add_f32") or op.startswith("v_mul_f32") or op.startswith("v_fmac_f32"):
            a, b = _src(expr, ops[1]), _src(expr, ops[2])
            if not bf16:
                a = f"e{a[1]}" if isinstance(a, tuple) and a[0] == "w" else a
                b = f"e{b[1]}" if isinstance(b, tuple) and b[0] == "w" else b
            if not (isinstance(a, str) and isinstance(b, str)):
                val = None
            elif op.startswith("v_add_f32"):
                val = canon_add(a, b)
            elif op.startswith("v_mul_f32"):
                val = f"({a}*{b})"
            else:
                acc = _src(expr, ops[0])
                acc = f"e{acc[1]}" if isinstance(acc, tuple) and acc[0] == "w" and not bf16 else acc
                val = f"fma({a},{b},{acc})" if isinstance(acc, str) else None
        else:
            val = None
        if d is not None and d[0] == "v":
            for k in range(d[1], d[2] + 1):
                expr[("v", k)] = val if k == d[1] else None
    for v in expr.values():
        if isinstance(v, str) and v.startswith("((L") and v.count("L") == 4:
            roots.append(v)
    return sorted(set(roots)) or None
