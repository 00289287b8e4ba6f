"""Functional CPU emulator of the gfx950 instructions the decode kernels use.

Test infrastructure: it runs the generated assembly of the decode kernels
(one workgroup of four 64-lane waves at a time) on host memory, so that the
kernels' control flow, addressing and numerics can be checked against the
oracle on the CPU.  It models what the kernels rely on and checks it
strictly:

  * global memory is a set of registered buffers; any access outside them
    raises Fault (on the GPU it would be a memory fault);
  * LDS accesses outside the workgroup's allocation raise Fault;
  * results of LDS, scalar and vector memory operations reach their
    destination only at the s_waitcnt that covers them (counters drain in
    issue order), so a value used before its wait reads stale data;
  * an LDS write becomes visible to the other waves only at such a wait too,
    so a barrier that is not preceded by the wait for the writes it should
    publish leaves them invisible;
  * waves run one at a time between barriers, in an order drawn from a seed,
    so that results that depend on the order expose a race.

Not modelled: instruction timing, the wait states the hardware asks for
between dependent MFMA / VALU / accvgpr instructions, and rounding inside the
MFMA (products and sums are taken in float64, the result rounded to fp32).
The layouts of the matrix, transposed-read and lane-swap instructions are the
ones the kernels' tile layout is built on: MFMA 16x16x32 A: lane l holds
row l % 16, k = 8 (l / 16) .. + 7; B: k = 8 (l / 16) .. + 7 of column l % 16;
D: rows 4 (l / 16) + i of column l % 16.
"""
from __future__ import annotations

import random
import re
import struct
from collections import deque

import numpy as np

M32 = 0xFFFFFFFF
M64 = (1 << 64) - 1


class Fault(Exception):
    """An access a GPU would fault on, or an instruction the emulator lacks."""


# ----------------------------------------------------------------- memory
class Memory:
    """Global memory: buffers at synthetic, widely spaced addresses."""

    def __init__(self):
        self.bufs = []
        self.next = 0x100000000

    def add(self, arr) -> int:
        data = np.ascontiguousarray(arr).reshape(-1).view(np.uint8).copy()
        base = self.next
        self.next += (data.size // (1 << 20) + 2) << 20
        self.bufs.append((base, data))
        return base

    def buffer(self, base) -> np.ndarray:
        for b, d in self.bufs:
            if b == base:
                return d
        raise KeyError(base)

    def _locate(self, lo, hi):
        for b, d in self.bufs:
            if b <= lo and hi <= b + d.size:
                return b, d
        raise Fault(f"global access [{lo:#x}, {hi:#x}) outside every buffer")

    def read(self, addrs, n):
        """addrs: int64 array of lane addresses -> uint8 [lanes, n]."""
        if addrs.size == 0:
            return np.zeros((0, n), np.uint8)
        b, d = self._locate(int(addrs.min()), int(addrs.max()) + n)
        idx = (addrs - b)[:, None] + np.arange(n)[None, :]
        return d[idx]

    def write(self, addrs, data):
        if addrs.size == 0:
            return
        n = data.shape[1]
        b, d = self._locate(int(addrs.min()), int(addrs.max()) + n)
        idx = (addrs - b)[:, None] + np.arange(n)[None, :]
        d[idx] = data

    def read_scalar(self, addr, ndw):
        b, d = self._locate(addr, addr + 4 * ndw)
        return [int(x) for x in d[addr - b:addr - b + 4 * ndw].view(np.uint32)]


# ----------------------------------------------------------------- parsing
_REG = re.compile(r"^(-?)([sva])(\d+)$|^(-?)([sva])\[(\d+):(\d+)\]$")


class Opd:
    __slots__ = ("kind", "idx", "n", "neg", "val", "abs")

    def __init__(self, kind, idx=0, n=1, neg=False, val=0, abs_=False):
        self.kind, self.idx, self.n, self.neg, self.val, self.abs = kind, idx, n, neg, val, abs_


def _float_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def parse_operand(tok):
    if len(tok) > 2 and tok[0] == "|" and tok[-1] == "|":     # |x|: absolute value (VOP3 float source)
        o = parse_operand(tok[1:-1])
        o.abs = True
        return o
    m = _REG.match(tok)
    if m:
        if m.group(2):
            return Opd(m.group(2), int(m.group(3)), 1, m.group(1) == "-")
        lo, hi = int(m.group(6)), int(m.group(7))
        return Opd(m.group(5), lo, hi - lo + 1, m.group(4) == "-")
    if tok in ("vcc", "exec", "m0", "scc"):
        return Opd(tok)
    if tok.startswith("."):
        return Opd("label")
    neg = tok.startswith("-") and not re.match(r"^-\d", tok)
    body = tok[1:] if neg else tok
    try:
        if re.match(r"^-?0x[0-9a-fA-F]+$", body):
            v = int(body, 16)
        elif re.match(r"^-?\d+$", body):
            v = int(body)
        else:
            v = _float_bits(float(body))
    except ValueError:
        raise Fault(f"operand not understood: {tok}")
    return Opd("imm", val=v, neg=neg)


class Instr:
    __slots__ = ("op", "args", "mods", "text")

    def __init__(self, text):
        self.text = text
        body = text.split(";")[0].strip()
        parts = body.split(None, 1)
        self.op = parts[0]
        self.args, self.mods = [], {}
        if len(parts) > 1:
            toks = [t.strip() for t in re.split(r",(?![^\[]*\])", parts[1])]
            last = toks[-1].split()
            toks[-1] = last[0]
            for m in last[1:]:
                if ":" in m:
                    k, v = m.split(":", 1)
                    self.mods[k] = v
                else:
                    self.mods[m] = True
            if self.op == "s_waitcnt":
                self.mods = {}
                for t in " ".join([parts[1]]).replace("&", " ").split():
                    mm = re.match(r"(vmcnt|lgkmcnt|expcnt)\((\d+)\)", t)
                    if mm:
                        self.mods[mm.group(1)] = int(mm.group(2))
                toks = []
            self.args = [parse_operand(t) for t in toks if t]


class Program:
    """The instruction list of one kernel in an assembly text, with its labels."""

    def __init__(self, text, kernel):
        lines = text.split("\n")
        start = None
        for i, line in enumerate(lines):
            if line.strip() == f"{kernel}:":
                start = i + 1
                break
        if start is None:
            raise KeyError(kernel)
        self.code, self.labels = [], {}
        for line in lines[start:]:
            s = line.strip()
            if not s or s.startswith(";"):
                continue
            if s.startswith(f".L{kernel}_end") or s.startswith(".Lfunc_end"):
                break
            if s.endswith(":"):
                self.labels[s[:-1]] = len(self.code)
                continue
            if s.startswith("."):
                continue
            self.code.append(Instr(s))
            if self.code[-1].op == "s_endpgm":
                pass


# ----------------------------------------------------------------- numerics
def f32(u):
    return np.asarray(u, np.uint32).view(np.float32)


def u32(f):
    return np.asarray(f, np.float32).view(np.uint32)


def bf16_to_f32(h):
    return (np.asarray(h, np.uint32) << 16).view(np.float32)


def f32_to_bf16_rne(x):
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, np.float32))
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) & 0xFFFF
    r = np.where(nan, (b >> 16) | 0x40, r)
    return r.astype(np.uint32)


def fmax_ieee(a, b):
    return np.where(np.isnan(a), b, np.where(np.isnan(b), a, np.maximum(a, b)))


def fmin_ieee(a, b):
    return np.where(np.isnan(a), b, np.where(np.isnan(b), a, np.minimum(a, b)))


# ----------------------------------------------------------------- waves
class Wave:
    def __init__(self, wg, wid):
        self.wg, self.wid = wg, wid
        self.s = [0] * 108
        self.vcc = 0
        self.exec = M64
        self.m0 = 0
        self.scc = 0
        self.v = np.zeros((512, 64), np.uint32)
        self.pc = 0
        self.lgkm = deque()
        self.vm = deque()
        self.state = "run"
        self.steps = 0
        self._em_bits, self._em = None, None
        self.store_data = None     # VGPRs a store of more than 64 bits read in the instruction before
        self.hist = deque(maxlen=6)  # (wait states it provides, VALU SGPR writes, VALU VGPR writes, M0 write, trans)

    # --- scalar operands
    def sget(self, o, width=32):
        if o.kind == "s":
            if width == 64:
                return self.s[o.idx] | (self.s[o.idx + 1] << 32)
            return self.s[o.idx]
        if o.kind == "imm":
            return o.val & (M64 if width == 64 else M32)
        if o.kind == "vcc":
            return self.vcc if width == 64 else self.vcc & M32
        if o.kind == "exec":
            return self.exec if width == 64 else self.exec & M32
        if o.kind == "m0":
            return self.m0
        if o.kind == "scc":
            return self.scc
        raise Fault(f"scalar operand kind {o.kind}")

    def sset(self, o, val, width=32):
        if o.kind == "s":
            self.s[o.idx] = val & M32
            if width == 64:
                self.s[o.idx + 1] = (val >> 32) & M32
        elif o.kind == "vcc":
            self.vcc = val & (M64 if width == 64 else M32)
        elif o.kind == "exec":
            self.exec = val & (M64 if width == 64 else M32)
        elif o.kind == "m0":
            self.m0 = val & M32
        else:
            raise Fault(f"scalar destination {o.kind}")

    # --- vector operands
    def vget(self, o, k=0):
        if o.kind == "v":
            r = self.v[o.idx + k].copy()
        elif o.kind == "a":
            r = self.v[256 + o.idx + k].copy()
        elif o.kind == "imm":
            r = np.full(64, o.val & M32, np.uint32)
        elif o.kind == "s":
            r = np.full(64, self.s[o.idx + k], np.uint32)
        elif o.kind == "vcc":
            r = np.full(64, self.vcc & M32, np.uint32)
        elif o.kind == "m0":
            r = np.full(64, self.m0, np.uint32)
        else:
            raise Fault(f"vector operand kind {o.kind}")
        return r

    def fget(self, o, k=0):
        x = f32(self.vget(o, k)).copy()
        if o.abs:
            x = np.abs(x)
        return -x if o.neg else x

    def execmask(self):
        if self._em_bits != self.exec:
            self._em_bits = self.exec
            self._em = _bits_to_mask(self.exec)
        return self._em

    def vset(self, o, val, k=0, mask=None):
        if mask is None:
            mask = self.execmask()
        base = o.idx + k + (256 if o.kind == "a" else 0)
        if o.kind not in ("v", "a"):
            raise Fault(f"vector destination {o.kind}")
        self.v[base][mask] = np.asarray(val, np.uint32)[mask]

    def lanes_bits(self, boolarr):
        return _mask_to_bits(self.execmask() & boolarr)

    # --- pending operations
    def drain(self, q, keep):
        while len(q) > keep:
            q.popleft()()

    def flush_lds_writes(self):
        """An LDS read is processed after this wave's earlier LDS operations:
        apply those writes now (their counter entries stay, as no-ops)."""
        for k, fn in enumerate(self.lgkm):
            if getattr(fn, "lds_write", False):
                fn()
                self.lgkm[k] = _noop


def _noop():
    pass


def _bits_to_mask(bits):
    b = np.frombuffer((bits & M64).to_bytes(8, "little"), np.uint8)
    return np.unpackbits(b, bitorder="little").astype(bool)


def _mask_to_bits(mask):
    return int.from_bytes(np.packbits(np.asarray(mask, bool), bitorder="little").tobytes(), "little")


_TRANS = ("v_exp_f32", "v_log_f32", "v_rcp_f32", "v_rsq_f32", "v_sqrt_f32", "v_sin_f32", "v_cos_f32")


def _regs(o):
    return set(range(o.idx, o.idx + o.n))


def check_wait_states(w, ins):
    """Wait states the hardware does not insert (software must, with s_nop or
    independent instructions; s_nop k gives k + 1):
      a VALU write of an SGPR read by a memory instruction as its address: 5;
      an SALU write of M0 read by a direct-to-LDS load as its LDS address: 1;
      a VALU write of a VGPR read by a DPP instruction: 2;
      a transcendental VALU result read by the next VALU: 1;
      a DOT result read by another VALU (not as a DOT's accumulator): 3.
    Raises Fault on a violation, then records the instruction."""
    op = ins.op
    def since(pred, limit):
        ws = 0
        for rec in reversed(w.hist):
            if ws >= limit:
                return False
            if pred(rec):
                return True
            ws += rec[0]
        return False
    if op.startswith(("global_", "buffer_")):
        for o in ins.args:
            if o.kind == "s":
                r = _regs(o)
                if since(lambda rec: rec[1] & r, 5):
                    raise Fault(f"s{o.idx} written by a VALU fewer than 5 wait states before its use as an address")
        if "_lds_" in op and since(lambda rec: rec[3], 1):
            raise Fault("M0 written by the instruction right before a direct-to-LDS load")
    if op.startswith("v_"):
        srcs = set()
        for o in ins.args[1:]:
            if o.kind == "v":
                srcs |= _regs(o)
        if op.endswith("_dpp") and since(lambda rec: rec[2] & srcs, 2):
            raise Fault("VGPR written by a VALU fewer than 2 wait states before a DPP read")
        if not op.startswith(_TRANS) and since(lambda rec: rec[4] and rec[2] & srcs, 1):
            raise Fault("transcendental result read by the next VALU (1 wait state needed)")
        # a DOT result read by another VALU instruction (a DOT of the same kind may
        # take it as its accumulator, srcC, at once)
        acc = _regs(ins.args[3]) if op.startswith("v_dot") and len(ins.args) > 3 and ins.args[3].kind == "v" \
            else set()
        if since(lambda rec: rec[5] and rec[2] & (srcs - acc), 3):
            raise Fault("DOT result read by another VALU fewer than 3 wait states later")
    # record
    nop = int(ins.args[0].val) + 1 if op == "s_nop" else 1
    sw, vw, m0, trans, dot = set(), set(), False, False, op.startswith("v_dot")
    if op.startswith("v_") and ins.args:
        d = ins.args[0]
        if d.kind == "s":
            sw = _regs(d)
        elif d.kind == "vcc":
            sw = {106, 107}
        elif d.kind == "v":
            vw = _regs(d)
        trans = op.startswith(_TRANS)
    elif op.startswith("s_") and ins.args and ins.args[0].kind == "m0":
        m0 = True
    w.hist.append((nop, sw, vw, m0, trans, dot))


class Workgroup:
    def __init__(self, prog, mem, lds_bytes, wg_id, kernarg, nwaves=4, seed=0, max_steps=5_000_000, hook=None):
        self.prog, self.mem, self.hook = prog, mem, hook
        self.lds = np.zeros(lds_bytes, np.uint8)
        self.waves = [Wave(self, w) for w in range(nwaves)]
        for w in self.waves:
            w.s[0], w.s[1] = kernarg & M32, kernarg >> 32
            w.s[2] = wg_id
            w.v[0] = np.arange(64, dtype=np.uint32) + 64 * w.wid
        self.rng = random.Random(seed)
        self.max_steps = max_steps

    def lds_check(self, addrs, n):
        if addrs.size and (int(addrs.min()) < 0 or int(addrs.max()) + n > self.lds.size):
            raise Fault(f"LDS access [{int(addrs.min())}, {int(addrs.max()) + n}) outside {self.lds.size} bytes")

    def run(self):
        while True:
            live = [w for w in self.waves if w.state != "done"]
            if not live:
                return
            order = live[:]
            self.rng.shuffle(order)
            for w in order:
                if w.state == "run":
                    self.step_until_block(w)
            live = [w for w in self.waves if w.state != "done"]
            if live and all(w.state == "barrier" for w in live):
                for w in live:
                    w.state = "run"

    def step_until_block(self, w):
        code = self.prog.code
        while w.state == "run":
            if w.pc >= len(code):
                raise Fault("ran past the end of the kernel")
            ins = code[w.pc]
            w.pc += 1
            w.steps += 1
            if w.steps > self.max_steps:
                raise Fault("step limit: the kernel does not terminate")
            if self.hook is not None:
                self.hook(self, w, w.pc - 1, ins)
            fn = OPS.get(ins.op)
            if fn is None:
                raise Fault(f"instruction not emulated: {ins.text}")
            # GCN store-data hazard: a VALU write of a VGPR that the previous
            # instruction, a store of more than 64 bits, reads as data needs one
            # wait state in between (the store may otherwise send the new value)
            if w.store_data is not None and ins.op.startswith("v_") and ins.args and ins.args[0].kind == "v":
                d = ins.args[0]
                lo, hi = w.store_data
                if d.idx <= hi and d.idx + d.n - 1 >= lo:
                    raise Fault(f"wave {w.wid} pc {w.pc - 1} '{ins.text}': writes v{d.idx} right after a store "
                                f"reading v[{lo}:{hi}] (store-data hazard)")
            w.store_data = None
            if ins.op.startswith(("global_store", "buffer_store")) and len(ins.args) > 1 and ins.args[1].kind == "v" \
                    and ins.args[1].n > 2:
                w.store_data = (ins.args[1].idx, ins.args[1].idx + ins.args[1].n - 1)
            check_wait_states(w, ins)
            try:
                fn(self, w, ins)
            except Fault as e:
                raise Fault(f"wave {w.wid} pc {w.pc - 1} '{ins.text}': {e}") from None


# ----------------------------------------------------------------- semantics
OPS = {}


def op(*names):
    def deco(fn):
        for n in names:
            OPS[n] = fn
        return fn
    return deco


def _sx32(x):
    x &= M32
    return x - (1 << 32) if x & 0x80000000 else x


@op("s_nop")
def _nop(g, w, i):
    pass


@op("s_endpgm")
def _end(g, w, i):
    w.drain(w.vm, 0)
    w.drain(w.lgkm, 0)
    w.state = "done"


@op("s_barrier")
def _barrier(g, w, i):
    w.state = "barrier"


@op("s_waitcnt")
def _waitcnt(g, w, i):
    if "vmcnt" in i.mods:
        w.drain(w.vm, i.mods["vmcnt"])
    if "lgkmcnt" in i.mods:
        w.drain(w.lgkm, i.mods["lgkmcnt"])


@op("s_branch")
def _branch(g, w, i):
    w.pc = g.prog.labels[i.text.split()[1]]


@op("s_cbranch_scc0", "s_cbranch_scc1")
def _cbranch(g, w, i):
    want = 1 if i.op.endswith("1") else 0
    if w.scc == want:
        w.pc = g.prog.labels[i.text.split()[1]]


@op("s_mov_b32")
def _smov(g, w, i):
    w.sset(i.args[0], w.sget(i.args[1]))


@op("s_mov_b64")
def _smov64(g, w, i):
    w.sset(i.args[0], w.sget(i.args[1], 64), 64)


def _s2(w, i):
    return w.sget(i.args[1]), w.sget(i.args[2])


@op("s_add_u32")
def _sadd(g, w, i):
    a, b = _s2(w, i)
    r = a + b
    w.scc = r >> 32
    w.sset(i.args[0], r)


@op("s_addc_u32")
def _saddc(g, w, i):
    a, b = _s2(w, i)
    r = a + b + w.scc
    w.scc = r >> 32
    w.sset(i.args[0], r)


@op("s_sub_u32")
def _ssub(g, w, i):
    a, b = _s2(w, i)
    w.scc = 1 if b > a else 0
    w.sset(i.args[0], a - b)


@op("s_add_i32", "s_sub_i32")
def _saddi(g, w, i):
    a, b = (_sx32(x) for x in _s2(w, i))
    r = a + b if i.op == "s_add_i32" else a - b
    w.scc = 1 if r > 0x7FFFFFFF or r < -0x80000000 else 0
    w.sset(i.args[0], r & M32)


@op("s_mul_i32")
def _smul(g, w, i):
    a, b = _s2(w, i)
    w.sset(i.args[0], (_sx32(a) * _sx32(b)) & M32)


@op("s_mul_hi_u32")
def _smulhi(g, w, i):
    a, b = _s2(w, i)
    w.sset(i.args[0], (a * b) >> 32)


@op("s_lshl_b32", "s_lshr_b32", "s_ashr_i32", "s_and_b32", "s_or_b32", "s_xor_b32")
def _sbit(g, w, i):
    a, b = _s2(w, i)
    if i.op == "s_lshl_b32":
        r = (a << (b & 31)) & M32
    elif i.op == "s_lshr_b32":
        r = a >> (b & 31)
    elif i.op == "s_ashr_i32":
        r = (_sx32(a) >> (b & 31)) & M32
    elif i.op == "s_and_b32":
        r = a & b
    elif i.op == "s_or_b32":
        r = a | b
    else:
        r = a ^ b
    w.scc = 1 if r else 0
    w.sset(i.args[0], r)


@op("s_lshl_b64", "s_lshr_b64", "s_or_b64", "s_and_b64")
def _sbit64(g, w, i):
    a = w.sget(i.args[1], 64)
    if i.op in ("s_lshl_b64", "s_lshr_b64"):
        b = w.sget(i.args[2]) & 63
        r = (a << b) & M64 if i.op == "s_lshl_b64" else a >> b
    else:
        b = w.sget(i.args[2], 64)
        r = a | b if i.op == "s_or_b64" else a & b
    w.scc = 1 if r else 0
    w.sset(i.args[0], r, 64)


@op("s_min_i32", "s_max_i32", "s_min_u32", "s_max_u32")
def _sminmax(g, w, i):
    a, b = _s2(w, i)
    if i.op.endswith("i32"):
        a2, b2 = _sx32(a), _sx32(b)
    else:
        a2, b2 = a, b
    if "min" in i.op:
        w.scc = 1 if a2 < b2 else 0
        r = a if a2 <= b2 else b
    else:
        w.scc = 1 if a2 > b2 else 0
        r = a if a2 >= b2 else b
    w.sset(i.args[0], r)


_CMP = {"eq": lambda a, b: a == b, "lg": lambda a, b: a != b, "lt": lambda a, b: a < b,
        "le": lambda a, b: a <= b, "gt": lambda a, b: a > b, "ge": lambda a, b: a >= b}


@op(*[f"s_cmp_{c}_{t}" for c in _CMP for t in ("i32", "u32")], "s_cmp_eq_u64", "s_cmp_lg_u64")
def _scmp(g, w, i):
    _, c, t = i.op.split("_")[1:]
    width = 64 if t == "u64" else 32
    a, b = w.sget(i.args[0], width), w.sget(i.args[1], width)
    if t == "i32":
        a, b = _sx32(a), _sx32(b)
    w.scc = 1 if _CMP[c](a, b) else 0


@op("s_bitcmp1_b32", "s_bitcmp0_b32")
def _sbitcmp(g, w, i):
    bit = (w.sget(i.args[0]) >> (w.sget(i.args[1]) & 31)) & 1
    w.scc = bit if i.op == "s_bitcmp1_b32" else 1 - bit


@op("s_cselect_b32")
def _scsel(g, w, i):
    w.sset(i.args[0], w.sget(i.args[1]) if w.scc else w.sget(i.args[2]))


@op("s_cselect_b64")
def _scsel64(g, w, i):
    w.sset(i.args[0], w.sget(i.args[1], 64) if w.scc else w.sget(i.args[2], 64), 64)


@op("s_ff1_i32_b32", "s_ff1_i32_b64")
def _sff1(g, w, i):
    width = 64 if i.op.endswith("64") else 32
    a = w.sget(i.args[1], width)
    r = (a & -a).bit_length() - 1 if a else -1
    w.sset(i.args[0], r & M32)


@op("s_and_saveexec_b64")
def _saveexec(g, w, i):
    src = w.sget(i.args[1], 64)
    w.sset(i.args[0], w.exec, 64)
    w.exec = src & w.exec
    w.scc = 1 if w.exec else 0


@op("s_load_dword", "s_load_dwordx2", "s_load_dwordx4", "s_load_dwordx8", "s_load_dwordx16")
def _sload(g, w, i):
    n = {"s_load_dword": 1, "s_load_dwordx2": 2, "s_load_dwordx4": 4, "s_load_dwordx8": 8, "s_load_dwordx16": 16}[i.op]
    base = w.sget(i.args[1], 64)
    off = w.sget(i.args[2]) if len(i.args) > 2 else 0
    vals = g.mem.read_scalar((base + off) & M64, n)
    dst = i.args[0]

    def land():
        for k in range(n):
            w.s[dst.idx + k] = vals[k]
    w.lgkm.append(land)


@op("s_memtime")
def _smemtime(g, w, i):
    now = w.steps

    def land():
        w.s[i.args[0].idx], w.s[i.args[0].idx + 1] = now & M32, 0
    w.lgkm.append(land)


@op("v_readfirstlane_b32")
def _rfl(g, w, i):
    src = w.vget(i.args[1])
    lane = (w.exec & -w.exec).bit_length() - 1 if w.exec else 0
    w.sset(i.args[0], int(src[lane]))


@op("v_readlane_b32")
def _rl(g, w, i):
    src = w.vget(i.args[1])
    w.sset(i.args[0], int(src[w.sget(i.args[2]) & 63]))


# --- VALU integer
def _vu(w, i, k):
    return w.vget(i.args[k]).astype(np.uint64)


@op("v_mov_b32")
def _vmov(g, w, i):
    w.vset(i.args[0], w.vget(i.args[1]))


@op("v_add_u32", "v_sub_u32", "v_and_b32", "v_or_b32", "v_xor_b32", "v_lshlrev_b32", "v_lshrrev_b32",
    "v_ashrrev_i32", "v_max_i32", "v_min_i32", "v_min_u32", "v_mul_u32_u24", "v_subrev_u32")
def _vint2(g, w, i):
    a, b = _vu(w, i, 1), _vu(w, i, 2)
    if i.op == "v_add_u32":
        r = a + b
    elif i.op == "v_sub_u32":
        r = a - b
    elif i.op == "v_subrev_u32":
        r = b - a
    elif i.op == "v_and_b32":
        r = a & b
    elif i.op == "v_or_b32":
        r = a | b
    elif i.op == "v_xor_b32":
        r = a ^ b
    elif i.op == "v_lshlrev_b32":
        r = b << (a & 31)
    elif i.op == "v_lshrrev_b32":
        r = b >> (a & 31)
    elif i.op == "v_ashrrev_i32":
        r = (b.astype(np.uint32).view(np.int32) >> (a & 31).astype(np.int32)).view(np.uint32).astype(np.uint64)
    elif i.op == "v_max_i32":
        r = np.maximum(a.astype(np.uint32).view(np.int32), b.astype(np.uint32).view(np.int32)).view(np.uint32)
    elif i.op == "v_min_i32":
        r = np.minimum(a.astype(np.uint32).view(np.int32), b.astype(np.uint32).view(np.int32)).view(np.uint32)
    elif i.op == "v_min_u32":
        r = np.minimum(a, b)
    else:
        r = (a & 0xFFFFFF) * (b & 0xFFFFFF)
    w.vset(i.args[0], (np.asarray(r, np.uint64) & M32).astype(np.uint32))


@op("v_lshl_add_u32", "v_lshl_or_b32", "v_bfe_u32", "v_or3_b32", "v_mad_i32_i24", "v_mad_u32_u24")
def _vint3(g, w, i):
    a, b, c = _vu(w, i, 1), _vu(w, i, 2), _vu(w, i, 3)
    if i.op == "v_lshl_add_u32":
        r = (a << (b & 31)) + c
    elif i.op == "v_lshl_or_b32":
        r = ((a << (b & 31)) & M32) | c
    elif i.op == "v_bfe_u32":
        r = (a >> (b & 31)) & ((np.uint64(1) << (c & 31)) - np.uint64(1))
    elif i.op == "v_or3_b32":
        r = a | b | c
    elif i.op == "v_mad_u32_u24":
        r = (a & 0xFFFFFF) * (b & 0xFFFFFF) + c
    else:
        def s24(x):
            x = (x & 0xFFFFFF).astype(np.int64)
            return np.where(x & 0x800000, x - (1 << 24), x)
        r = (s24(a) * s24(b) + c.astype(np.uint32).view(np.int32).astype(np.int64)).astype(np.uint64)
    w.vset(i.args[0], (np.asarray(r).astype(np.uint64) & M32).astype(np.uint32))


@op("v_add_u32_dpp")
def _vdpp(g, w, i):
    """v_add_u32 with a DPP-permuted first source (row_shr / row_bcast)."""
    src0, src1 = w.vget(i.args[1]), w.vget(i.args[2])
    dst_old = w.vget(i.args[0])
    lanes = np.arange(64)
    ok = np.ones(64, bool)
    perm = lanes.copy()
    if "row_shr" in i.mods:
        n = int(i.mods["row_shr"])
        perm = lanes - n
        ok = (lanes % 16) >= n
    elif "row_bcast" in i.mods:
        n = int(i.mods["row_bcast"])
        if n == 15:
            perm = (lanes // 16) * 16 - 1
            ok = lanes >= 16
        else:
            perm = np.full(64, 31)
            ok = lanes >= 32
    else:
        raise Fault(f"dpp control not emulated: {i.text}")
    row_mask = int(i.mods.get("row_mask", "0xf"), 0)
    bank_mask = int(i.mods.get("bank_mask", "0xf"), 0)
    bound = "bound_ctrl" in i.mods
    v0 = np.where(ok, src0[np.clip(perm, 0, 63)], 0).astype(np.uint64)
    write = ((row_mask >> (lanes // 16)) & 1).astype(bool) & ((bank_mask >> ((lanes // 4) % 4)) & 1).astype(bool)
    if not bound:
        write &= ok
    r = ((v0 + src1.astype(np.uint64)) & M32).astype(np.uint32)
    w.vset(i.args[0], np.where(write, r, dst_old), mask=w.execmask())


@op("v_permlane16_swap_b32", "v_permlane32_swap_b32")
def _vswap(g, w, i):
    a, b = w.vget(i.args[0]), w.vget(i.args[1])
    na, nb = a.copy(), b.copy()
    if i.op == "v_permlane32_swap_b32":
        na[32:], nb[:32] = b[:32], a[32:]
    else:
        for r in (0, 2):
            na[16 * (r + 1):16 * (r + 2)] = b[16 * r:16 * (r + 1)]
            nb[16 * r:16 * (r + 1)] = a[16 * (r + 1):16 * (r + 2)]
    w.vset(i.args[0], na)
    w.vset(i.args[1], nb)


# --- VALU float
def _fset(w, i, x):
    with np.errstate(all="ignore"):
        w.vset(i.args[0], u32(np.asarray(x, np.float32)))


@op("v_add_f32", "v_sub_f32", "v_mul_f32", "v_max_f32", "v_min_f32")
def _vf2(g, w, i):
    a, b = w.fget(i.args[1]), w.fget(i.args[2])
    with np.errstate(all="ignore"):
        if i.op == "v_add_f32":
            r = a + b
        elif i.op == "v_sub_f32":
            r = a - b
        elif i.op == "v_mul_f32":
            r = a * b
        elif i.op == "v_max_f32":
            r = fmax_ieee(a, b)
        else:
            r = fmin_ieee(a, b)
    _fset(w, i, r)


@op("v_fma_f32", "v_max3_f32")
def _vf3(g, w, i):
    a, b, c = w.fget(i.args[1]), w.fget(i.args[2]), w.fget(i.args[3])
    with np.errstate(all="ignore"):
        if i.op == "v_fma_f32":
            r = (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)
        else:
            r = fmax_ieee(fmax_ieee(a, b), c)
    _fset(w, i, r)


@op("v_exp_f32", "v_log_f32", "v_rcp_f32")
def _vtrans(g, w, i):
    a = w.fget(i.args[1])
    with np.errstate(all="ignore"):
        if i.op == "v_exp_f32":
            r = np.exp2(a.astype(np.float64))
        elif i.op == "v_log_f32":
            r = np.log2(a.astype(np.float64))
        else:
            r = 1.0 / a.astype(np.float64)
        r = r.astype(np.float32)
    _fset(w, i, r)


@op("v_dot2_f32_bf16")
def _vdot2bf16(g, w, i):
    """D = a.lo * b.lo + a.hi * b.hi + c, a and b bf16 pairs, c fp32; computed
    exactly and rounded once to fp32."""
    a, b = w.vget(i.args[1]), w.vget(i.args[2])
    c = w.fget(i.args[3]).astype(np.float64)
    bf = lambda x: ((x & 0xFFFF) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    with np.errstate(all="ignore"):
        r = bf(a) * bf(b) + bf(a >> 16) * bf(b >> 16) + c
    _fset(w, i, r.astype(np.float32))


@op("v_cvt_pk_f16_f32")
def _vcvtpkf16(g, w, i):
    """Two fp32 -> two fp16 (round to nearest even, IEEE overflow to inf), packed."""
    with np.errstate(all="ignore"):
        lo = w.fget(i.args[1]).astype(np.float16).view(np.uint16).astype(np.uint32)
        hi = w.fget(i.args[2]).astype(np.float16).view(np.uint16).astype(np.uint32)
    w.vset(i.args[0], (lo | (hi << 16)).astype(np.uint32))


@op("v_cvt_pk_bf16_f32")
def _vcvtpk(g, w, i):
    lo, hi = f32_to_bf16_rne(w.fget(i.args[1])), f32_to_bf16_rne(w.fget(i.args[2]))
    w.vset(i.args[0], (lo | (hi << 16)).astype(np.uint32))


def e4m3_to_f32(b):
    """OCP E4M3 byte -> float32 (exact): 1 sign, 4 exponent (bias 7), 3
    mantissa bits, subnormals at exponent 0, NaN at S.1111.111, no inf."""
    b = np.asarray(b, np.uint32)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e.astype(np.float64) - 7))
    val = np.where((e == 15) & ((b & 7) == 7), np.nan, val)
    return (sign * val).astype(np.float32)


@op("v_cvt_scalef32_pk_bf16_fp8")
def _vcvt_fp8(g, w, i):
    """Two e4m3 bytes of src0 (bytes 0, 1; op_sel[0]: bytes 2, 3) times the
    fp32 scale -> two bf16 (round to nearest even) packed into the destination."""
    src = w.vget(i.args[1])
    scale = w.fget(i.args[2])
    hi_sel = i.mods.get("op_sel", "[0,0,0]").strip("[]").split(",")[0] == "1"
    sh = 16 if hi_sel else 0
    lo = e4m3_to_f32((src >> sh) & 0xFF) * scale
    hi = e4m3_to_f32((src >> (sh + 8)) & 0xFF) * scale
    w.vset(i.args[0], (f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16)).astype(np.uint32))


@op(*[f"v_cmp_{c}_{t}" for c in ("eq", "lt", "gt", "le", "ge", "lg", "ne") for t in ("f32", "i32", "u32")])
def _vcmp(g, w, i):
    _, c, t = i.op.split("_")[1:]
    if t == "f32":
        a, b = w.fget(i.args[1]), w.fget(i.args[2])
    elif t == "i32":
        a, b = w.vget(i.args[1]).view(np.int32), w.vget(i.args[2]).view(np.int32)
    else:
        a, b = w.vget(i.args[1]), w.vget(i.args[2])
    fn = {"eq": np.equal, "lt": np.less, "gt": np.greater, "le": np.less_equal, "ge": np.greater_equal,
          "lg": np.not_equal, "ne": np.not_equal}[c]
    with np.errstate(all="ignore"):
        res = fn(a, b)
    bits = w.lanes_bits(res)
    dst = i.args[0]
    if dst.kind == "vcc":
        w.vcc = bits
    else:
        w.sset(dst, bits, 64)


@op("v_cndmask_b32")
def _vcnd(g, w, i):
    a, b = w.vget(i.args[1]), w.vget(i.args[2])
    sel = i.args[3]
    bits = w.vcc if sel.kind == "vcc" else w.sget(sel, 64)
    m = _bits_to_mask(bits)
    w.vset(i.args[0], np.where(m, b, a))


@op("v_accvgpr_read_b32", "v_accvgpr_write_b32")
def _vacc(g, w, i):
    w.vset(i.args[0], w.vget(i.args[1]), mask=np.ones(64, bool))


_LANES = np.arange(64)
_M, _KG = _LANES % 16, _LANES // 16


@op("v_mfma_f32_16x16x32_bf16")
def _mfma(g, w, i):
    d, a, b, c = i.args
    ra = np.stack([w.vget(a, k) for k in range(4)])        # [4, 64]
    rb = np.stack([w.vget(b, k) for k in range(4)])
    va = bf16_to_f32(np.stack([ra & 0xFFFF, ra >> 16], axis=1).reshape(8, 64)).astype(np.float64)
    vb = bf16_to_f32(np.stack([rb & 0xFFFF, rb >> 16], axis=1).reshape(8, 64)).astype(np.float64)
    kl = np.arange(8)[:, None]
    A = np.zeros((16, 32))
    B = np.zeros((32, 16))
    A[_M[None, :], 8 * _KG[None, :] + kl] = va
    B[8 * _KG[None, :] + kl, _M[None, :]] = vb
    C = np.zeros((16, 16))
    if c.kind != "imm":
        rc = np.stack([w.vget(c, k) for k in range(4)])
        C[4 * _KG[None, :] + np.arange(4)[:, None], _M[None, :]] = f32(rc).astype(np.float64)
    with np.errstate(all="ignore"):
        D = (A @ B + C).astype(np.float32)
    out = D[4 * _KG[None, :] + np.arange(4)[:, None], _M[None, :]]      # [4, 64]
    full = np.ones(64, bool)
    for r in range(4):
        w.vset(d, u32(out[r]), k=r, mask=full)


# --- LDS
def _lds_addr(w, i):
    off = int(i.mods.get("offset", 0))
    return w.vget(i.args[1] if i.op.startswith("ds_read") else i.args[0]).astype(np.int64) + off


@op("ds_read_b32", "ds_read_b64", "ds_read_b128", "ds_read_b64_tr_b16")
def _dsread(g, w, i):
    w.flush_lds_writes()
    mask = w.execmask()
    addr = _lds_addr(w, i)
    n = {"ds_read_b32": 4, "ds_read_b64": 8, "ds_read_b128": 16, "ds_read_b64_tr_b16": 8}[i.op]
    g.lds_check(addr[mask], n)
    data = np.zeros((64, n), np.uint8)
    idx = addr[mask][:, None] + np.arange(n)[None, :]
    data[mask] = g.lds[idx]
    words = data.view(np.uint32)                    # [64, n/4]
    if i.op == "ds_read_b64_tr_b16":
        # 4 x 4 transpose of 16-bit values inside each group of 16 lanes:
        # lane j of group g receives element j & 3 of lanes 4r + (j >> 2), r = 0..3
        h = data.view(np.uint16).reshape(4, 16, 4)  # [group, lane, elem]
        j, r = np.arange(16)[:, None], np.arange(4)[None, :]
        out = h[:, 4 * r + (j >> 2), j & 3]
        words = np.ascontiguousarray(out).reshape(64, 4).view(np.uint32)
    dst = i.args[0]
    vals = words.copy()

    def land():
        for k in range(vals.shape[1]):
            w.vset(dst, vals[:, k], k=k, mask=mask)
    w.lgkm.append(land)


@op("ds_write_b32", "ds_write_b64", "ds_write_b128")
def _dswrite(g, w, i):
    mask = w.execmask()
    addr = _lds_addr(w, i)
    n = {"ds_write_b32": 4, "ds_write_b64": 8, "ds_write_b128": 16}[i.op]
    g.lds_check(addr[mask], n)
    src = i.args[1]
    data = np.stack([w.vget(src, k) for k in range(n // 4)], axis=1).copy().view(np.uint8)   # [64, n]
    am = addr[mask]
    dm = data[mask]

    def land():
        g.lds[am[:, None] + np.arange(n)[None, :]] = dm
    land.lds_write = True
    w.lgkm.append(land)


# --- global memory
def _gaddr(w, i, vidx, sidx):
    off = int(i.mods.get("offset", 0))
    base = w.sget(i.args[sidx], 64)
    return (w.vget(i.args[vidx]).astype(np.int64) + base + off)


@op("global_load_dword", "global_load_dwordx4")
def _gload(g, w, i):
    n = 4 if i.op == "global_load_dword" else 16
    mask = w.execmask()
    addr = _gaddr(w, i, 1, 2)
    data = np.zeros((64, n), np.uint8)
    data[mask] = g.mem.read(addr[mask], n)
    words = data.view(np.uint32).copy()
    dst = i.args[0]

    def land():
        for k in range(words.shape[1]):
            w.vset(dst, words[:, k], k=k, mask=mask)
    w.vm.append(land)


@op("global_store_dword", "global_store_dwordx2", "global_store_dwordx4")
def _gstore(g, w, i):
    n = {"global_store_dword": 4, "global_store_dwordx2": 8, "global_store_dwordx4": 16}[i.op]
    mask = w.execmask()
    addr = _gaddr(w, i, 0, 2)
    data = np.stack([w.vget(i.args[1], k) for k in range(n // 4)], axis=1).copy().view(np.uint8)
    g.mem.write(addr[mask], data[mask])
    w.vm.append(lambda: None)


@op("global_load_lds_dwordx4")
def _gload_lds(g, w, i):
    mask = w.execmask()
    addr = _gaddr(w, i, 0, 1)
    data = g.mem.read(addr[mask], 16)
    lanes = np.nonzero(mask)[0]
    dst = w.m0 + int(i.mods.get("offset", 0)) + 16 * lanes
    g.lds_check(dst.astype(np.int64), 16)

    def land():
        g.lds[dst[:, None] + np.arange(16)[None, :]] = data
    w.vm.append(land)


# ----------------------------------------------------------------- launch
def run_kernel(text, kernel, lds_bytes, mem, kernarg_bytes, grid, seed=0, nwaves=4, hook=None):
    """Run every workgroup of a launch (one after the other)."""
    prog = Program(text, kernel)
    karg = mem.add(np.frombuffer(kernarg_bytes, np.uint8))
    for wg in range(grid):
        Workgroup(prog, mem, lds_bytes, wg, karg, nwaves=nwaves, seed=seed * 1000003 + wg, hook=hook).run()
