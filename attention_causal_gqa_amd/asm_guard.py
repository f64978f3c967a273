"""Build-time check of the inline-assembly loads in compiled device code.

A kernel may issue a global load from inline assembly so that the
compiler's wait-count insertion does not see it (and so does not drain it
early); the kernel then waits for it itself with ``s_waitcnt vmcnt(N)``.
The compiler, however, believes the asm statement's output registers hold
their value as soon as the statement is issued.  Between the issue and the
wait that retires the load, any instruction the compiler places that reads
those registers (a copy, a spill, a reuse) sees stale data, and any
instruction that writes them is later overwritten when the data lands.
Either is a silent wrong result.

``hazards(asm_text)`` reports every instruction that touches a register of a
possibly in-flight inline-assembly load, on any path through each
function's control-flow graph.  Vector memory operations retire in issue
order, so ``vmcnt(N)`` retires a load once at least N younger vector memory
operations have been issued after it.  The analysis is a forward data flow:
for each pending load (identified by its instruction) it keeps the fewest
younger operations issued since it, over every path reaching a point, and a
load counts as pending if it is pending on any path.

Paths the kernel cannot take are told apart only through wave-uniform
scalar conditions, which the compiler materialises as flags and tests again
later (for example "wait in one arm of a branch, then branch again on the
same condition").  Each path carries the truth values it has learnt of
integer comparisons of unchanged operands and the symbolic lane masks built
from them (``s_cselect``, ``v_cmp`` of uniform operands, ``v_cndmask`` 0/1
images, ``s_and``/``s_andn2``/``s_xor`` with exec), and a conditional branch
whose condition is known on a path takes only the matching successor.
Everything else is treated as unknown, so an unrecognised idiom can only
add reports, never hide one.  Values are versioned by the instruction that
defines them; at a loop header the facts about values the loop defines are
dropped (the next iteration defines them anew) and the others kept.  A
vector memory operation is counted as issued only where some lane is known
to be active.
"""

import re

BRANCH_OPS = ("s_branch", "s_cbranch_")
# Operations that certainly count in vmcnt on gfx9 (loads, stores and atomics
# of the vector memory path).  Cache-control operations are left out: counting
# an operation that does not count would credit a wait with retiring a load
# it does not retire.
VMEM_OPS = ("global_load", "global_store", "global_atomic", "buffer_load", "buffer_store", "buffer_atomic",
            "flat_load", "flat_store", "flat_atomic", "scratch_load", "scratch_store")
YOUNGER_CAP = 64
MAX_STATES = 256  # path-distinct states kept per block before they are merged

# Instructions whose first operand is read, not written.
_NO_DEST = ("s_cmp", "s_bitcmp", "s_cbranch", "s_branch", "s_waitcnt", "s_nop", "s_barrier", "s_setprio",
            "s_sleep", "s_sendmsg", "s_endpgm", "s_trap", "s_dcache", "s_icache", "s_setreg", "s_ttrace",
            "global_store", "buffer_store", "flat_store", "scratch_store", "ds_write", "ds_store",
            "global_load_lds", "buffer_wbl2", "buffer_inv", "exp ")
# Scalar instructions that leave SCC alone.
_NO_SCC = ("s_mov", "s_cmov", "s_cselect", "s_cbranch", "s_branch", "s_waitcnt", "s_nop", "s_barrier",
           "s_setprio", "s_sleep", "s_sendmsg", "s_load", "s_buffer_load", "s_getpc", "s_endpgm", "s_dcache",
           "s_icache", "s_setreg", "s_getreg")
_INT_TYPES = ("i16", "u16", "i32", "u32", "i64", "u64")
_SPECIAL = {"vcc": (106, 107), "vcc_lo": (106,), "vcc_hi": (107,), "exec": (126, 127), "exec_lo": (126,),
            "exec_hi": (127,), "m0": ("m0",), "scc": ("scc",)}


def vregs(text):
    """VGPRs and AGPRs named in an operand list, as (file, index) pairs."""
    out = set()
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b", text):
        if m.group(1):
            out |= {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _sreg_tuple(tok):
    """The scalar registers one operand names, or None if it names none."""
    tok = tok.strip()
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return tuple(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"s(\d+)", tok)
    if m:
        return (int(m.group(1)),)
    return _SPECIAL.get(tok)


def _vreg_tuple(tok):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok.strip())
    if m:
        return tuple(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", tok.strip())
    return (int(m.group(1)),) if m else None


def _is_imm(tok):
    return re.fullmatch(r"-?(0x[0-9a-fA-F]+|\d+)", tok.strip()) is not None


def functions(asm_text):
    """Device assembly -> {function: [block, ...]}, a block being {"label", "ins": [(op, operands, in_asm,
    text)]}.  A block ends at a label or after a branch or s_endpgm."""
    funcs, blocks, in_asm, cur = {}, None, False, None
    for line in asm_text.splitlines():
        raw = line.strip()
        if raw.startswith(".amdgpu_metadata"):
            break
        if raw.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if raw.startswith(";;#ASMEND"):
            in_asm = False
            continue
        s = line.split(";")[0].strip()
        if not s:
            continue
        if s.endswith(":") and " " not in s:
            if not s.startswith("."):  # a function (or data) symbol
                blocks = funcs.setdefault(s[:-1], [])
                cur = {"label": None, "ins": []}
                blocks.append(cur)
            elif blocks is not None:
                cur = {"label": s[:-1], "ins": []}
                blocks.append(cur)
            continue
        if s.startswith(".") or cur is None:
            continue
        op, _, rest = s.partition(" ")
        if cur["ins"] and cur["ins"][-1][0].startswith(BRANCH_OPS + ("s_endpgm",)):
            cur = {"label": None, "ins": []}
            blocks.append(cur)
        ops = [t.strip() for t in rest.split(",")] if rest.strip() else []
        cur["ins"].append((op, ops, in_asm, s))
    return funcs


def successors(blocks):
    index = {b["label"]: i for i, b in enumerate(blocks) if b["label"]}
    succ = []
    for i, b in enumerate(blocks):
        last = b["ins"][-1] if b["ins"] else None
        nxt = [i + 1] if i + 1 < len(blocks) else []
        if last is None:
            succ.append(nxt)
        elif last[0] == "s_endpgm":
            succ.append([])
        elif last[0].startswith(("s_setpc", "s_swappc")):
            raise ValueError(f"indirect branch not supported by the check: {last[3]}")
        elif last[0] == "s_branch":
            succ.append([index[last[1][0].split()[0]]])
        elif last[0].startswith("s_cbranch_"):
            succ.append([index[last[1][0].split()[0]]] + nxt)
        else:
            succ.append(nxt)
    return succ


def _scalar_liveness(blocks, succ):
    """Scalar registers (numbers) each block may read before writing them, over all paths from its start
    (VCC as 106-107, SCC as "scc").  Only used to forget dead flags, so erring either way is safe."""
    gen, kill = [], []
    for b in blocks:
        g, kl = set(), set()
        for op, ops, _, _ in b["ins"]:
            w = {r for r in writes(op, ops) if isinstance(r, int)}
            reads = set()
            srcs = ops if (op.startswith(_NO_DEST) or (op.startswith("v_cmp") and "_e32" in op)) else ops[1:]
            for t in srcs:
                reads |= set(r for r in (_sreg_tuple(t) or ()) if isinstance(r, int))
            if op in ("s_cbranch_vccz", "s_cbranch_vccnz") or op.startswith(("v_cndmask_b32_e32", "v_addc",
                                                                          "v_subb", "v_div_fmas")):
                reads |= {106, 107}
            if op.startswith(("s_cbranch_scc", "s_cselect", "s_cmov", "s_addc", "s_subb")):
                reads.add("scc")
            g |= reads - kl
            kl |= w
            if op.startswith("s_") and not op.startswith(_NO_SCC):
                kl.add("scc")
        gen.append(g)
        kill.append(kl)
    live = [set() for _ in blocks]
    changed = True
    while changed:
        changed = False
        for i in range(len(blocks) - 1, -1, -1):
            out = set().union(*[live[j] for j in succ[i]]) if succ[i] else set()
            new = gen[i] | (out - kill[i])
            if new != live[i]:
                live[i] = new
                changed = True
    return live


def _loops(succ):
    """{header: blocks of its loop}: a back edge u -> h (h still on the depth-first search stack) closes a
    loop made of h and every block that reaches u without passing through h."""
    back, state, stack = [], {0: 1}, [(0, iter(succ[0]) if succ else iter(()))]
    while stack:
        node, it = stack[-1]
        nxt = next(it, None)
        if nxt is None:
            state[node] = 2
            stack.pop()
        elif state.get(nxt) == 1:
            back.append((node, nxt))
        elif nxt not in state:
            state[nxt] = 1
            stack.append((nxt, iter(succ[nxt])))
    pred = {}
    for u, vs in enumerate(succ):
        for v in vs:
            pred.setdefault(v, []).append(u)
    loops = {}
    for u, h in back:
        body = loops.setdefault(h, {h})
        work = [u]
        while work:
            x = work.pop()
            if x in body:
                continue
            body.add(x)
            work.extend(pred.get(x, []))
    return loops


def writes(op, ops):
    """Registers an instruction may write: scalar registers as numbers, vector ones as ("v"/"a", n).
    Errs towards more (the first operand of anything not known to read it)."""
    written = set()
    if ops and not op.startswith(_NO_DEST) and not (op.startswith("v_cmp") and "_e32" in op):
        written |= set(_sreg_tuple(ops[0]) or ()) | vregs(ops[0])
    if len(ops) > 1 and ("_co_" in op or op.startswith(("v_mad_u64", "v_mad_i64", "v_div_scale"))):
        written |= set(_sreg_tuple(ops[1]) or ())
    if op.startswith("v_cmp") and "_e32" in op:
        written |= {106, 107}
    if op.startswith("v_cmpx") or "saveexec" in op:
        written |= {126, 127}
    if "swap" in op:  # v_swap, v_permlane*_swap: every register operand
        for t in ops:
            written |= set(_sreg_tuple(t) or ()) | vregs(t)
    return written


# ---- symbolic scalar state ------------------------------------------------
# A literal is True (always), False (never), (atom, polarity), ("and", l1, l2)
# (both hold; at most four atoms) or ("not", l) (l fails).  A lane mask
# is ("zero",), ("uni", lit, E) = lit ? lanes of E : none, ("nuni", lit, E) =
# its complement, or absent (unknown).  E is an exec token: "ALL" (every
# lane), ("e0",) (the lanes the wave started with), or a token from an exec
# write, with a parent when it is known to be a subset of another.


def _neg(lit):
    if lit is True or lit is False:
        return not lit
    if lit[0] == "not":
        return lit[1]
    if lit[0] == "and":
        return ("not", lit)
    return (lit[0], not lit[1])


def _conj(a, b):
    """The literal a and b (conjunctions of at most four comparisons; None beyond)."""
    if a is False or b is False:
        return False
    if a is True:
        return b
    if b is True or a == b:
        return a
    lit = ("and", a, b)
    return lit if len(_atoms_in(lit, set())) <= 4 else None


class _State:
    __slots__ = ("pending", "facts", "ver", "epoch", "masks", "scc", "vuni", "vbool", "exec", "nonempty")

    def __init__(self):
        self.pending = {}    # site -> (younger, regs)
        self.facts = {}      # atom -> bool
        self.ver = {}        # register -> version token
        self.epoch = ("entry",)
        self.masks = {}      # tuple of sregs -> mask
        self.scc = None      # literal or None
        self.vuni = {}       # vgpr -> (value id, part, exec token): same value in the lanes of that exec
        self.vbool = {}      # vgpr -> (literal, exec token): 1 if literal else 0 in the lanes of that exec
        self.exec = ("e0",)
        self.nonempty = frozenset({("e0",), "ALL"})

    def copy(self):
        s = _State()
        s.pending = dict(self.pending)
        s.facts = dict(self.facts)
        s.ver = dict(self.ver)
        s.epoch = self.epoch
        s.masks = dict(self.masks)
        s.scc = self.scc
        s.vuni = dict(self.vuni)
        s.vbool = dict(self.vbool)
        s.exec = self.exec
        s.nonempty = self.nonempty
        return s

    def key(self):
        """Paths are kept apart by the facts a live flag refers to and by flags set to a constant (those
        decide the branches the compiler lowers through flags); other facts are joined by intersection."""
        live = set()
        for v in self.masks.values():
            _atoms_in(v, live)
        _atoms_in(self.scc, live)
        for v in self.vbool.values():
            _atoms_in(v, live)
        consts = frozenset((d, v) for d, v in self.masks.items() if v == ("zero",) or v == ("uni", True, "ALL"))
        return frozenset((a, v) for a, v in self.facts.items() if a in live) | consts

    def version(self, reg):
        return self.ver.get(reg, (self.epoch, reg))


class _Analysis:
    def __init__(self, blocks):
        self.blocks = blocks
        self.succ = successors(blocks)
        self.loops = _loops(self.succ)
        self.headers = set(self.loops)
        self.live_in = _scalar_liveness(blocks, self.succ)
        # scalar registers each loop may write
        self.loop_writes = {h: {r for b in body for ins in blocks[b]["ins"] for r in writes(ins[0], ins[1])
                                if isinstance(r, int)} for h, body in self.loops.items()}

    # exec token relations: a token made by an exec write carries, as its
    # last element, a token known to contain it (or None)
    def subset(self, a, b):
        if b == "ALL" or a == b:
            return True
        while _up(a) is not None:
            a = _up(a)
            if a == b:
                return True
        return False

    def truth(self, st, lit):
        """True, False or None (unknown) for a literal on the path whose facts are st.facts."""
        if lit is True or lit is False:
            return lit
        if lit[0] == "not":
            t = self.truth(st, lit[1])
            return None if t is None else not t
        if lit[0] == "and":
            ta, tb = self.truth(st, lit[1]), self.truth(st, lit[2])
            if ta is False or tb is False:
                return False
            return True if (ta is True and tb is True) else None
        v = st.facts.get(lit[0])
        return None if v is None else v == lit[1]

    def learn(self, st, lit, val):
        """Record on st what `lit` having truth `val` implies about single comparisons."""
        if lit is True or lit is False:
            return
        if lit[0] == "not":
            self.learn(st, lit[1], not val)
        elif lit[0] == "and":
            if val:
                self.learn(st, lit[1], True)
                self.learn(st, lit[2], True)
            elif self.truth(st, lit[1]) is True:
                self.learn(st, lit[2], False)
            elif self.truth(st, lit[2]) is True:
                self.learn(st, lit[1], False)
        elif st.facts.get(lit[0]) is None:
            st.facts[lit[0]] = lit[1] == val

    # operand values
    def value_id(self, st, tok):
        """An identifier of an operand's wave-uniform value (equal ids, equal values), or None."""
        tok = tok.strip()
        if _is_imm(tok):
            return ("imm", int(tok, 0))
        regs = _sreg_tuple(tok)
        if regs is not None and all(isinstance(r, int) for r in regs):
            return ("s",) + tuple((r, st.version(r)) for r in regs)
        vr = _vreg_tuple(tok)
        if vr is not None:
            ent = [st.vuni.get(r) for r in vr]
            if all(e is not None for e in ent) and len({(e[0], e[2]) for e in ent}) == 1 \
                    and [e[1] for e in ent] == list(range(len(vr))) and self.subset(st.exec, ent[0][2]):
                return ent[0][0]
        return None

    def mask_of(self, st, tok):
        tok = tok.strip()
        if tok == "exec":
            return ("uni", True, st.exec)
        if _is_imm(tok):
            v = int(tok, 0)
            return ("zero",) if v == 0 else ("uni", True, "ALL") if v == -1 else None
        regs = _sreg_tuple(tok)
        return st.masks.get(regs) if regs is not None else None

    def m_not(self, m):
        if m is None or m[0] == "sub":
            return None
        if m[0] == "zero":
            return ("uni", True, "ALL")
        if m[0] == "uni":
            return ("zero",) if (m[1] is True and m[2] == "ALL") else ("nuni", m[1], m[2])
        return ("uni", m[1], m[2])

    def m_and(self, a, b):
        if a is None or b is None:
            if a == ("zero",) or b == ("zero",):
                return ("zero",)
            known = a if b is None else b
            return ("sub", self.ub(known)) if known is not None and self.ub(known) != "ALL" else None
        if a[0] == "zero" or b[0] == "zero":
            return ("zero",)
        if a[0] == "sub" or b[0] == "sub":
            return self.m_sub(a, b, larger=False)
        if a[0] == "nuni" and b[0] == "uni":
            a, b = b, a
        if a[0] == "uni" and b[0] == "uni":
            if self.subset(a[2], b[2]):
                inner, outer = a, b
            elif self.subset(b[2], a[2]):
                inner, outer = b, a
            else:
                return None
            lit = _conj(inner[1], outer[1])
            if lit is None:
                return ("sub", inner[2])
            return ("zero",) if lit is False else ("uni", lit, inner[2])
        if a[0] == "uni" and b[0] == "nuni":
            # lanes(Ea) if la, minus (lanes(Eb) if lb)
            if a[1] is True and self.subset(a[2], b[2]):
                return ("uni", _neg(b[1]), a[2]) if b[1] is not True else ("zero",)
            if a[1] == b[1] and self.subset(a[2], b[2]):
                return ("zero",)
        return self.m_sub(a, b, larger=False)

    def m_or(self, a, b):
        if a == ("zero",):
            return b
        if b == ("zero",):
            return a
        return self.m_sub(a, b, larger=True)

    def ub(self, m):
        """An exec token whose lanes include every lane of mask m ("ALL" if none is known)."""
        if m is None or m[0] == "nuni":
            return "ALL"
        if m[0] == "zero":
            return None
        return m[2] if m[0] == "uni" else m[1]

    def m_sub(self, a, b, larger):
        """("sub", E) for a result contained in the larger (union) or smaller (intersection) of the two
        masks' bounds, when those are nested."""
        ea, eb = self.ub(a), self.ub(b)
        if ea is None or eb is None:
            e = eb if ea is None else ea
            return ("zero",) if (e is None or not larger) else ("sub", e)
        if self.subset(ea, eb):
            return ("sub", eb if larger else ea)
        if self.subset(eb, ea):
            return ("sub", ea if larger else eb)
        return None

    # the step function
    def step(self, st, bi, k, op, ops, text):
        """Apply one (non-branch) instruction's scalar effects to st."""
        new_masks, new_scc, new_vbool, new_vuni = {}, None, {}, {}
        scc_written = op.startswith("s_") and not op.startswith(_NO_SCC)
        # comparisons
        m = re.match(r"(s|v)_cmpk?_(lt|le|gt|ge|eq|lg|ne)_([iu]\d+)", op)
        atom_lit = None
        if m and m.group(3) in _INT_TYPES:
            kind, typ = m.group(2), m.group(3)
            srcs = ops[-2:] if len(ops) >= 2 else []
            ids = [self.value_id(st, t) for t in srcs]
            if len(ids) == 2 and None not in ids:
                a, b = ids
                if kind in ("gt", "le"):
                    a, b = b, a
                if kind in ("lt", "gt"):
                    atom_lit = (("lt", typ, a, b), True)
                elif kind in ("le", "ge"):  # a <= b  is  not (b < a)  (a, b already swapped for le)
                    atom_lit = (("lt", typ, a, b), False)
                else:
                    x, y = sorted([a, b], key=repr)
                    atom_lit = (("eq", typ, x, y), kind == "eq")
        if op.startswith("s_cmp"):
            new_scc = atom_lit
            scc_written = True
        elif op.startswith("v_cmp") and not op.startswith("v_cmpx"):
            dest = ("vcc" if "_e32" in op else ops[0]) if ops else None
            dregs = _sreg_tuple(dest) if dest else None
            val = None
            if atom_lit is not None:
                val = ("uni", atom_lit, st.exec)
            else:
                # v_cmp_{eq,ne}_u32 of a 0/1 image against 0 or 1
                mm = re.match(r"v_cmp_(eq|ne|lg)_[iu]32", op)
                if mm and len(ops) >= 2:
                    srcs = ops[-2:]
                    for vi, ci in ((0, 1), (1, 0)):
                        vr = _vreg_tuple(srcs[vi])
                        if vr and len(vr) == 1 and _is_imm(srcs[ci]) and int(srcs[ci], 0) in (0, 1):
                            img = st.vbool.get(vr[0])
                            if img is not None and self.subset(st.exec, img[1]):
                                lit = img[0] if (int(srcs[ci], 0) == 1) == (mm.group(1) == "eq") else _neg(img[0])
                                val = ("uni", lit, st.exec) if lit is not False else ("zero",)
                            break
            if val is None:
                val = ("sub", st.exec)  # a per-lane result: some of the active lanes
            if dregs is not None:
                new_masks[dregs] = val
        elif op == "s_cselect_b64" and len(ops) == 3:
            if st.scc is not None and _is_imm(ops[1]) and _is_imm(ops[2]):
                t, f = int(ops[1], 0), int(ops[2], 0)
                if (t, f) == (-1, 0):
                    new_masks[_sreg_tuple(ops[0])] = ("uni", st.scc, "ALL")
                elif (t, f) == (0, -1):
                    new_masks[_sreg_tuple(ops[0])] = ("uni", _neg(st.scc), "ALL")
        elif op in ("s_mov_b64", "s_and_b64", "s_andn2_b64", "s_or_b64", "s_xor_b64", "s_not_b64",
                    "s_orn2_b64") and ops and ops[0] != "exec":
            d = _sreg_tuple(ops[0])
            srcs = [self.mask_of(st, t) for t in ops[1:]]
            val = None
            if op == "s_mov_b64":
                val = srcs[0]
            elif op == "s_not_b64":
                val = self.m_not(srcs[0])
            elif op == "s_and_b64":
                val = self.m_and(srcs[0], srcs[1])
            elif op == "s_andn2_b64":
                val = self.m_and(srcs[0], self.m_not(srcs[1]))
            elif op == "s_or_b64":
                val = self.m_or(srcs[0], srcs[1])
            elif op == "s_orn2_b64":
                val = self.m_or(srcs[0], self.m_not(srcs[1]))
            elif op == "s_xor_b64":
                if ops[2] == "-1":
                    val = self.m_not(srcs[0])
                elif ops[1] == "-1":
                    val = self.m_not(srcs[1])
            if d is not None and val is not None:
                new_masks[d] = val
        elif op == "v_cndmask_b32_e64" and len(ops) == 4 and ops[1] == "0" and ops[2] == "1":
            mk = self.mask_of(st, ops[3])
            vr = _vreg_tuple(ops[0])
            if vr and mk is not None:
                if mk[0] == "zero":
                    new_vbool[vr[0]] = (False, st.exec)
                elif mk[0] == "uni" and self.subset(st.exec, mk[2]):
                    new_vbool[vr[0]] = (mk[1], st.exec)
        elif op in ("v_mov_b32_e32", "v_mov_b64_e32") and len(ops) == 2:
            vr = _vreg_tuple(ops[0])
            vid = self.value_id(st, ops[1])
            if vr and vid is not None:
                for part, r in enumerate(vr):
                    new_vuni[r] = (vid, part, st.exec)

        # exec writes
        new_exec = None
        if "saveexec" in op or (ops and ops[0] in ("exec", "exec_lo", "exec_hi")) or op.startswith("v_cmpx"):
            token = ("x", bi, k, None)
            src = self.mask_of(st, ops[1]) if len(ops) > 1 else None
            if op in ("s_and_saveexec_b64",) or (op in ("s_and_b64", "s_andn2_b64") and "exec" in ops[1:2]) \
                    or op.startswith("v_cmpx"):
                new_exec = ("x", bi, k, st.exec)
            elif op in ("s_or_b64", "s_or_saveexec_b64", "s_xor_b64"):
                # exec | S (or exec ^ S): within the larger of the two when they are nested.
                if op == "s_or_saveexec_b64":
                    other = ops[1] if len(ops) > 1 else None
                else:
                    other = ops[2] if ops[1:2] == ["exec"] else ops[1] if ops[2:3] == ["exec"] else None
                om = self.mask_of(st, other) if other else None
                e = self.ub(om) if other else "ALL"
                if op != "s_xor_b64" and om is not None and om[0] == "uni" and om[1] is True \
                        and self.subset(st.exec, om[2]):
                    new_exec = om[2]  # restoring a saved mask that contains the current one
                elif op != "s_xor_b64" and e is None:
                    new_exec = st.exec  # S is empty
                elif e is not None and self.subset(e, st.exec) and op != "s_xor_b64":
                    new_exec = st.exec  # S within the current lanes
                else:
                    if e is not None and self.subset(st.exec, e) and e != "ALL":
                        token = ("x", bi, k, e)
                    new_exec = token
            elif op == "s_mov_b64" and src is not None and src[0] == "uni" and src[1] is True:
                new_exec = src[2]
            elif op in ("s_mov_b64", "s_andn2_saveexec_b64") and src is not None and self.ub(src) not in (None, "ALL"):
                new_exec = ("x", bi, k, self.ub(src))
            else:
                new_exec = token
            if "saveexec" in op and ops:
                new_masks[_sreg_tuple(ops[0])] = ("uni", True, st.exec)

        written = writes(op, ops)
        for r in written:
            if isinstance(r, int):
                st.ver[r] = ("d", bi, k, r)
            elif isinstance(r, tuple) and r[0] == "v":
                st.vuni.pop(r[1], None)
                st.vbool.pop(r[1], None)
            elif isinstance(r, tuple) and r[0] == "a":
                pass
        if written:
            sw = {r for r in written if isinstance(r, int)}
            st.masks = {d: v for d, v in st.masks.items() if not (set(d) & sw)}
        if scc_written:
            st.scc = new_scc
        st.masks.update({d: v for d, v in new_masks.items() if d is not None})
        st.vbool.update(new_vbool)
        st.vuni.update(new_vuni)
        if new_exec is not None:
            st.exec = new_exec

    def branch_targets(self, st, bi):
        """[(successor, state)] of block bi's end, pruning successors the path's facts rule out."""
        blk = self.blocks[bi]
        nexts = self.succ[bi]
        last = blk["ins"][-1] if blk["ins"] else None
        if last is None or not last[0].startswith("s_cbranch_") or len(nexts) != 2:
            return [(j, st) for j in nexts]
        taken, fall = nexts
        cond = last[0][len("s_cbranch_"):]
        out = []

        def add(j, lit, val, extra_nonempty=None):
            # Follow edge j on which `lit` has truth `val` (lit None: no condition learnt).
            if lit is not None:
                t = self.truth(st, lit)
                if t is not None and t != val:
                    return
            s2 = st.copy()
            if lit is not None and self.truth(st, lit) is None:
                self.learn(s2, lit, val)
            if extra_nonempty is not None:
                s2.nonempty = s2.nonempty | {extra_nonempty}
            out.append((j, s2))

        if cond in ("vccnz", "vccz"):
            m = st.masks.get((106, 107))
            nz = cond == "vccnz"  # taken when VCC is non-zero
            if m is not None and m[0] == "zero":
                out.append((fall, st) if nz else (taken, st))
                return out
            if m is not None and m[0] == "uni" and m[2] in st.nonempty:
                add(taken, m[1], nz)
                add(fall, m[1], not nz)
                return out
            return [(taken, st.copy()), (fall, st.copy())]
        if cond in ("scc0", "scc1"):
            if st.scc is not None:
                add(taken, st.scc, cond == "scc1")
                add(fall, st.scc, cond != "scc1")
                return out
            return [(taken, st.copy()), (fall, st.copy())]
        if cond in ("execz", "execnz"):
            if st.exec in st.nonempty:
                # exec is known to hold a lane on this path (for example the
                # wave's whole mask, which the structurizer tests again after
                # a uniform branch's arm): the execz edge cannot be taken
                return [(fall, st.copy())] if cond == "execz" else [(taken, st.copy())]
            s_nz = st.copy()
            s_nz.nonempty = s_nz.nonempty | {st.exec}
            return [(taken, st.copy() if cond == "execz" else s_nz), (fall, s_nz if cond == "execz" else st.copy())]
        return [(taken, st.copy()), (fall, st.copy())]


def _merge(an, a, b, j):
    """Join of two states with equal facts, at block j."""
    m = a.copy()
    m.facts = {f: v for f, v in a.facts.items() if b.facts.get(f) == v}
    for site, (y, regs) in b.pending.items():
        m.pending[site] = (min(y, a.pending[site][0]), regs) if site in a.pending else (y, regs)
    keys = set(a.ver) | set(b.ver)
    epoch = a.epoch if a.epoch == b.epoch else ("phi", j)
    m.epoch = epoch
    m.ver = {}
    for r in keys:
        va, vb = a.version(r), b.version(r)
        m.ver[r] = va if va == vb else ("phi", j, r)
    m.masks = {}
    for d in set(a.masks) & set(b.masks):
        va, vb = a.masks[d], b.masks[d]
        v = va if va == vb else an.m_sub(va, vb, larger=True)
        if v is not None and v != ("sub", "ALL"):
            m.masks[d] = v
    m.scc = a.scc if a.scc == b.scc else None
    m.vuni = {}
    for r in set(a.vuni) & set(b.vuni):
        va, vb = a.vuni[r], b.vuni[r]
        if va == vb:
            m.vuni[r] = va
        elif va[1:] == vb[1:] and _current(a, va[0]) is not None and _current(a, va[0]) == _current(b, vb[0]):
            # on both paths the register holds the current value of the same scalar registers
            m.vuni[r] = (("s",) + tuple((x, m.version(x)) for x in _current(a, va[0])),) + va[1:]
    m.vbool = {r: v for r, v in a.vbool.items() if b.vbool.get(r) == v}
    if a.exec == b.exec:
        m.exec = a.exec
    else:
        # the union of two exec masks lies within their nearest common ancestor
        anc, e = [a.exec], a.exec
        while _up(e) is not None:
            e = _up(e)
            anc.append(e)
        e = b.exec
        while e not in anc and _up(e) is not None:
            e = _up(e)
        m.exec = ("phi", j, None, e if e in anc else None)
    m.nonempty = a.nonempty & b.nonempty
    return m


def _current(st, vid):
    """The scalar registers whose present values a value id names, or None."""
    if vid[0] != "s" or any(st.version(r) != v for r, v in vid[1:]):
        return None
    return tuple(r for r, _ in vid[1:])


def _same(a, b):
    return (a.pending == b.pending and a.ver == b.ver and a.epoch == b.epoch and a.masks == b.masks
            and a.scc == b.scc and a.vuni == b.vuni and a.vbool == b.vbool and a.exec == b.exec
            and a.nonempty == b.nonempty)


def _defined_in(obj, body, hdr=None):
    """Whether a fact, mask or value (nested tuples) names a version or exec token made inside `body`.
    With hdr = (j, W), a join inside the loop of a register outside W (those the loop never writes) counts
    as made before the loop: whichever path reached the join, the register still holds its value from the
    loop's entry, so every iteration of one run of the loop sees that same value."""
    if isinstance(obj, tuple):
        if len(obj) >= 2 and obj[0] in ("d", "phi", "hdr", "x", "many") and isinstance(obj[1], int):
            if (hdr is not None and obj[0] == "phi" and len(obj) == 3
                    and isinstance(obj[2], int) and obj[2] not in hdr[1]):
                return False
            return obj[1] in body
        return any(_defined_in(o, body, hdr) for o in obj)
    return False


def _at_header(an, st, j):
    """Entering loop header j: the values the loop defines are about to be defined again, so every path fact
    that names one of them (or an exec token made in the loop) is dropped, and the registers the loop writes
    take a version of the header's own.  Facts about values from before the loop stay true."""
    body, hdr = an.loops[j], (j, an.loop_writes[j])
    s = st.copy()
    for r in an.loop_writes[j]:
        s.ver[r] = ("hdr", j, r)
    s.facts = {a: v for a, v in s.facts.items() if not _defined_in(a, body, hdr)}
    masks = {}
    for d, v in s.masks.items():
        if not _defined_in(v, body, hdr):
            masks[d] = v  # the value on this edge, made before the loop
        else:
            # keep only a bound from before the loop: the lanes of an exec
            # mask that contains every exec mask the loop makes
            e = _outside(an, an.ub(v), body)
            if e not in (None, "ALL"):
                masks[d] = ("sub", e)
    s.masks = masks
    s.scc = None
    s.vuni = {r: v for r, v in s.vuni.items() if not _defined_in(v, body, hdr)}
    s.vbool = {r: v for r, v in s.vbool.items() if not _defined_in(v, body, hdr)}
    if _defined_in(s.exec, body):
        s.exec = ("hdr", j, "exec", _outside(an, s.exec, body))
        s.nonempty = frozenset(x for x in s.nonempty if not _defined_in(x, body))
    return s


def _outside(an, tok, body):
    """The nearest of tok and its known supersets that is not made inside `body`, or None."""
    while tok is not None and _defined_in(tok, body):
        tok = _up(tok)
    return tok


def _up(tok):
    """The token an exec token is known to lie within, or None."""
    return tok[3] if isinstance(tok, tuple) and len(tok) == 4 and tok[0] in ("x", "phi", "hdr") else None


def _atoms_in(obj, out):
    if isinstance(obj, tuple):
        if len(obj) == 4 and obj[0] in ("lt", "eq") and isinstance(obj[1], str):
            out.add(obj)
        else:
            for o in obj:
                _atoms_in(o, out)
    return out


def _relevant(st):
    """Drop the facts that can no longer decide a branch: those about atoms that no live flag refers to and
    whose operands have been overwritten (so that no later comparison can produce the same atom)."""
    live = set()
    for v in st.masks.values():
        _atoms_in(v, live)
    _atoms_in(st.scc, live)
    for v in st.vbool.values():
        _atoms_in(v, live)

    def current(vid):
        if vid[0] != "s":
            return True
        return all(st.version(r) == ver for r, ver in vid[1:])

    st.facts = {a: v for a, v in st.facts.items() if a in live or (current(a[2]) and current(a[3]))}
    return st


def _forget(st, j):
    """The state with no path facts and flags (too many distinct paths reach block j)."""
    s = st.copy()
    s.facts = {}
    s.masks = {d: v for d, v in s.masks.items() if not _atoms_in(v, set())}
    s.scc = None
    s.vbool = {}
    return s


def hazards(asm_text, allowed=(), workers=1):
    """Reports "function: instruction" for every instruction that may touch a register of an in-flight
    inline-assembly load, except those listed in `allowed`.  Functions are checked in `workers` processes."""
    funcs = [(f, b) for f, b in functions(asm_text).items() if any(ins[2] for blk in b for ins in blk["ins"])]
    if workers > 1 and len(funcs) > 1:
        import concurrent.futures
        with concurrent.futures.ProcessPoolExecutor(min(workers, len(funcs))) as ex:
            results = list(ex.map(_function_hazards, funcs))
    else:
        results = [_function_hazards(fb) for fb in funcs]
    allowed = set(allowed)
    return [p for r in results for p in r if p not in allowed]


def _function_hazards(func_blocks):
    func, blocks = func_blocks
    problems = []
    an = _Analysis(blocks)
    entry = [dict() for _ in blocks]  # block -> {facts key: state}
    st0 = _State()
    entry[0][st0.key()] = st0
    work = [(0, st0.key())]
    found = set()
    while work:
        i, key = work.pop()
        if key not in entry[i]:
            continue
        st = entry[i][key].copy()
        for k, (op, ops, in_asm, text) in enumerate(blocks[i]["ins"]):
            if op.startswith(BRANCH_OPS):
                continue
            if op == "s_waitcnt":
                m = re.search(r"vmcnt\((\d+)\)", " ".join(ops))
                if m:
                    n = int(m.group(1))
                    st.pending = {s: v for s, v in st.pending.items() if v[0] < n}
                continue
            touched = vregs(", ".join(ops))
            is_vmem = op.startswith(VMEM_OPS)
            is_asm_load = in_asm and op.startswith(("global_load", "buffer_load")) and "lds" not in op
            live = set()
            for _, (_, regs) in st.pending.items():
                live |= regs
            if is_asm_load and ops:
                # The destination may be a register of an older pending
                # load of the same registers (loads land in issue order);
                # the address operands may not.
                dest = vregs(ops[0])
                clash = (touched - dest) & live
            else:
                dest, clash = set(), touched & live
            if clash and (i, k) not in found:
                found.add((i, k))
                problems.append(f"{func}: {text}")
            if is_vmem and st.exec in st.nonempty:
                # (with no lane active, the operation might not be
                # issued: it is not counted)
                st.pending = {s: (min(v[0] + 1, YOUNGER_CAP), v[1]) for s, v in st.pending.items()}
                if is_asm_load:
                    st.pending[(i, k)] = (0, dest)
            an.step(st, i, k, op, ops, text)
        for j, s2 in an.branch_targets(st, i):
            if j in an.headers:
                s2 = _at_header(an, s2, j)
            live = an.live_in[j]
            s2.masks = {d: v for d, v in s2.masks.items() if set(d) & live}
            if "scc" not in live:
                s2.scc = None
            s2 = _relevant(s2)
            kj = s2.key()
            if kj not in entry[j] and len(entry[j]) >= MAX_STATES:
                s2 = _forget(s2, j)
                kj = s2.key()
            old = entry[j].get(kj)
            new = s2 if old is None else _merge(an, old, s2, j)
            if old is None or not _same(old, new):
                entry[j][kj] = new
                work.append((j, kj))
    return problems
