"""Host-side checks of the decode kernels' LDS and global addressing.

The assembly generator's load, dequantize and read sequences are run on the
CPU (the fp8 kernel's by a small symbolic interpreter, the bf16 kernel's by
the emulator of tests/gcn_emu.py) and the data they move is compared with the
tile layout the kernels rely on: a page tile is 9 x 8 blocks of 1 KB (a half
page tile 9 x 4); block (K, R) holds rows 8R..8R+7 and 16-byte chunks
8K..8K+7; row r sits at 128 (r % 8) in its block and chunk c at
16 ((c % 8) ^ tp(r)), tp(r) = t(r % 8) ^ 2 ((r / 8) % 2), t(q) = 2 (q & 3) + (q >> 2).
"""
import os
import re
import sys

import pytest

sys.path.insert(0, os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                "mla_latent_kv_39_amd", "csrc"))
import gen_decode_gfx950 as G  # noqa: E402


def _t(q):
    return ((q & 3) << 1) | (q >> 2)


def _tp(r):
    return _t(r & 7) ^ (2 * ((r >> 3) & 1))


def tile_byte(r, c):
    return (8 * (c // 8) + r // 8) * 1024 + ((r % 8) * 8 + ((c % 8) ^ _tp(r))) * 16


ZERO = ("zero",)


class Wave:
    """Per-lane interpreter.  VGPR values are ints (addresses) or tuples of
    symbolic bytes; LDS maps byte address -> symbolic byte."""

    def __init__(self, wave, lds):
        self.v, self.s, self.lds = {}, {G.S_WAVE: wave}, lds
        self.exec = (1 << 64) - 1
        self.vcc = [False] * 64
        self.masks = {}
        self.reads, self.writes, self.loads = [], {}, []
        for L in range(64):
            self.v[(G.V_LANE, L)] = L
            self.v[(G.V_G, L)] = L >> 4
            self.v[(G.V_R16, L)] = L & 15

    def sval(self, x):
        x = x.strip()
        if x == "m0":
            return self.s["m0"]
        m = re.fullmatch(r"s(\d+)", x)
        if m:
            return self.s[int(m.group(1))]
        m = re.fullmatch(r"s\[(\d+):\d+\]", x)
        if m:
            return self.s[int(m.group(1))]
        return 1.0 if x == "1.0" else int(x, 0)

    def val(self, x, L):
        m = re.fullmatch(r"v(\d+)", x.strip())
        return self.v[(int(m.group(1)), L)] if m else self.sval(x)

    def run(self, lines):
        for ln in lines:
            st = ln.strip()
            if not st or st.startswith(";") or st.endswith(":"):
                continue
            op, _, rest = st.partition(" ")
            args = [a.strip() for a in re.split(r",(?![^\[]*\])", rest)]
            if op in ("s_nop", "s_waitcnt", "s_barrier"):
                continue
            if op.startswith("s_"):
                self.scalar(op, args)
            else:
                for L in range(64):
                    if (self.exec >> L) & 1:
                        self.vector(op, args, L)

    def scalar(self, op, a):
        if op == "s_mov_b64" and a[0] == "exec":
            self.exec = (1 << 64) - 1 if a[1] == "-1" else int(a[1], 0)
            return
        key = "m0" if a[0] == "m0" else int(re.fullmatch(r"s(\d+)", a[0]).group(1))
        x = [self.sval(v) for v in a[1:]]
        self.s[key] = {"s_mul_i32": lambda: x[0] * x[1], "s_add_u32": lambda: x[0] + x[1],
                       "s_addc_u32": lambda: x[0] + x[1], "s_lshl_b32": lambda: x[0] << x[1],
                       "s_lshr_b32": lambda: x[0] >> x[1], "s_and_b32": lambda: x[0] & x[1],
                       "s_mov_b32": lambda: x[0]}[op]()

    def vector(self, op, a, L):
        V = lambda i: self.val(a[i], L)
        dst = lambda: int(re.fullmatch(r"v(\d+)", a[0]).group(1))
        arith = {"v_lshlrev_b32": lambda: V(2) << V(1), "v_lshrrev_b32": lambda: V(2) >> V(1),
                 "v_and_b32": lambda: V(1) & V(2), "v_xor_b32": lambda: V(1) ^ V(2),
                 "v_add_u32": lambda: V(1) + V(2), "v_mul_u32_u24": lambda: V(1) * V(2),
                 "v_lshl_add_u32": lambda: (V(1) << V(2)) + V(3), "v_lshl_or_b32": lambda: (V(1) << V(2)) | V(3),
                 "v_bfe_u32": lambda: (V(1) >> V(2)) & ((1 << V(3)) - 1), "v_mov_b32": lambda: V(1)}
        if op in arith and all(isinstance(V(k), (int, float)) for k in range(1, len(a))):
            self.v[(dst(), L)] = arith[op]()
        elif op in arith or op in ("v_rcp_f32", "v_sub_f32", "v_cvt_pk_bf16_f32"):
            # arithmetic on loaded data: kept symbolic, with its operands
            self.v[(dst(), L)] = ("op", op) + tuple(V(k) for k in range(1, len(a)))
        elif op == "v_cmp_lt_f32":
            self.vcc[L] = True          # data-dependent (scale > 0): both outcomes keep the sources
        elif op == "v_cmp_gt_i32":
            if a[0] == "vcc":
                self.vcc[L] = V(1) > V(2)
            else:
                self.masks.setdefault(a[0], [False] * 64)[L] = V(1) > V(2)
        elif op == "v_cndmask_b32":
            keep = self.vcc[L] if a[3] == "vcc" else self.masks[a[3]][L]
            if isinstance(V(2), int) and isinstance(V(1), int):
                self.v[(dst(), L)] = V(2) if keep else V(1)
            else:
                self.v[(dst(), L)] = V(2) if keep else (ZERO,) * 4
        elif op == "v_cvt_scalef32_pk_bf16_fp8":
            src = V(1)
            pair = src[2:4] if "op_sel:[1,0,0]" in " ".join(a) else src[0:2]
            self.v[(dst(), L)] = ("bf16",) + tuple(pair)
        elif op in ("ds_read_b32", "ds_read_b64", "ds_read_b128", "ds_read_b64_tr_b16"):
            base, _, off = a[1].partition(" offset:")
            addr = self.val(base, L) + int(off or 0)
            self.reads.append((op, addr, L))
            if op != "ds_read_b64_tr_b16":
                n = {"ds_read_b32": 4, "ds_read_b64": 8, "ds_read_b128": 16}[op]
                m = re.match(r"v\[(\d+):", a[0]) or re.fullmatch(r"v(\d+)", a[0])
                d0 = int(m.group(1))
                byts = [self.lds.get(addr + b, ("undef",)) for b in range(n)]
                for q in range(n // 4):
                    self.v[(d0 + q, L)] = tuple(byts[4 * q:4 * q + 4])
        elif op in ("ds_write_b128", "ds_write_b64", "ds_write_b32"):
            src, _, off = a[1].partition(" offset:")
            addr = self.val(a[0], L) + int(off or 0)
            if op == "ds_write_b32":
                self.writes[addr] = self.val(src, L)
            else:
                d0 = int(re.match(r"v\[(\d+):", src).group(1))
                for q in range(4 if op == "ds_write_b128" else 2):
                    self.writes[addr + 4 * q] = self.v[(d0 + q, L)]
        elif op == "global_load_lds_dwordx4":
            src = V(0) + self.sval(a[1])
            dst_addr = self.s["m0"] + 16 * L
            self.loads.append((src, dst_addr))
            for b in range(16):
                self.lds[dst_addr + b] = ("g", src + b)
        else:
            raise AssertionError(f"instruction not modelled: {op}")


def _leaves(x):
    """The symbolic source bytes (("g", address) or ZERO) a value derives from."""
    if isinstance(x, tuple) and x and x[0] == "g":
        return {x}
    if x == ZERO:
        return {ZERO}
    out = set()
    if isinstance(x, (tuple, list)) or hasattr(x, "__iter__") and not isinstance(x, str):
        for y in x:
            if isinstance(y, (tuple, list)) or hasattr(y, "__iter__") and not isinstance(y, str):
                out |= _leaves(y)
    return out


def lines_of(fn, *args):
    a = G.Asm()
    fn(a, *args)
    return a.lines


@pytest.fixture
def bf16_mode():
    G.configure(False)
    yield
    G.configure(False)


@pytest.fixture
def fp8_mode():
    G.configure(True)
    yield
    G.configure(False)


# ---------------------------------------------------------------- bf16 kernel
# The bf16 kernel works on half pages: a tile is 9 x 4 blocks of 1 KB, block
# (K, R) at (4K + R) KB, with the same row / chunk swizzle inside a block.
# These checks run the generated instructions on the emulator of
# tests/gcn_emu.py and look at the data each lane ends up with.
import numpy as np  # noqa: E402

import gcn_emu as E  # noqa: E402


def half_byte(r, c):
    return (4 * (c // 8) + r // 8) * 1024 + ((r % 8) * 8 + ((c % 8) ^ _tp(r))) * 16


def _workgroup(lines, mem):
    text = "k:\n" + "\n".join(lines) + "\n\ts_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_endpgm\n"
    wg = E.Workgroup(E.Program(text, "k"), mem, G.P_BASE + G.P_BYTES, 0, mem.add(np.zeros(16, np.uint8)))
    lanes = np.arange(64, dtype=np.uint32)
    for w in wg.waves:
        w.s[G.S_WAVE] = w.wid
        w.v[G.V_LANE], w.v[G.V_G], w.v[G.V_R16] = lanes, lanes >> 4, lanes & 15
    return wg


def _lane_setup():
    a = G.Asm()
    G.lane_constants(a)
    G.lane_constants_hp(a)
    return a.lines


@pytest.mark.parametrize("half", [0, 1])
@pytest.mark.parametrize("valid", [64, 40, 33, 9, 1])
def test_bf16_half_page_loads(bf16_mode, half, valid):
    """Tile chunk (r, c) of the half page holds page row 32 half + r, chunk c
    (row 32 half for rows past the data); all loads stay inside the page."""
    page = np.zeros((64, 72, 4), np.uint32)
    page[..., 0] = np.arange(64)[:, None]
    page[..., 1] = np.arange(72)[None, :]
    page[..., 2] = 0xA5A5A5A5
    mem = E.Memory()
    base = mem.add(page)
    step = 6 + half
    a = G.Asm()
    G.dma_setup_hp(a, half, G.S_TMP + 8)
    for g in G.dma_groups_hp():
        a.lines += g
    wg = _workgroup(_lane_setup() + a.lines, mem)
    for w in wg.waves:
        w.s[G.S_PAGE], w.s[G.S_PAGE + 1] = base & 0xFFFFFFFF, base >> 32
        w.s[G.S_NVALID], w.s[G.S_TMP + 8] = valid, step
    wg.run()
    tile = wg.lds[(step & 3) * G.HS_BYTES:((step & 3) + 1) * G.HS_BYTES]
    for r in range(32):
        src = 32 * half + r if 32 * half + r < valid else 32 * half
        for c in range(72):
            got = tile[half_byte(r, c):half_byte(r, c) + 16].view(np.uint32)
            assert (got[0], got[1], got[2]) == (src, c, 0xA5A5A5A5), (r, c, got)


def test_bf16_half_tile_reads(bf16_mode):
    """Score reads: lane (g, r16) of fragment (ks, tb) gets row 16tb + r16,
    chunk 4ks + g.  Output reads of wave w, column block cb: lane (g, j) gets
    column 128w + 16cb + j of rows 4g .. 4g+3 (first read) and 16 + 4g ..
    (second read)."""
    slot = 2
    mem = E.Memory()
    lines = _lane_setup()
    T = G.S_TMP
    lines += [f"\ts_mov_b32 s{T}, {slot * G.HS_BYTES}",
              f"\tv_add_u32 v{G.V_UQ}, s{T}, v{G.V_QKE}", f"\tv_add_u32 v{G.V_UQ + 1}, s{T}, v{G.V_QKO}"]
    lines += [f"\tv_add_u32 v{G.V_UP + m}, s{T}, v{G.V_PVM[m]}" for m in range(4)]
    wg = _workgroup(lines, mem)
    wg.run()
    # tile element (row, col) holds the bf16 bit pattern row * 576 + col
    for r in range(32):
        for c in range(72):
            off = slot * G.HS_BYTES + half_byte(r, c)
            wg.lds[off:off + 16] = np.arange(r * 576 + 8 * c, r * 576 + 8 * c + 8, dtype=np.uint16).view(np.uint8)
    for w in wg.waves:
        for i in range(36):
            ks, tb = divmod(i, 2)
            prog = E.Program("k:\n" + G.qk_read_hp(i)[0].format(buf="v[16:19]") + "\n\ts_waitcnt lgkmcnt(0)\n", "k")
            for ins in prog.code:
                E.OPS[ins.op](wg, w, ins)
            got = w.v[16:20].T.copy().view(np.uint16)            # [lane, 8]
            lanes = np.arange(64)
            want = ((16 * tb + (lanes & 15)) * 576 + 8 * (4 * ks + (lanes >> 4)))[:, None] + np.arange(8)[None, :]
            assert np.array_equal(got, want.astype(np.uint16)), (w.wid, i)
        for cb in range(8):
            reads = [x.format(lo="v[20:21]", hi="v[22:23]") for x in G.pv_read_hp(cb)]
            prog = E.Program("k:\n" + "\n".join(reads) + "\n\ts_waitcnt lgkmcnt(0)\n", "k")
            for ins in prog.code:
                E.OPS[ins.op](wg, w, ins)
            got = w.v[20:24].T.copy().view(np.uint16)             # [lane, 8]: rows 4g+r, then 16+4g+r
            lanes = np.arange(64)
            col = 128 * w.wid + 16 * cb + (lanes & 15)
            rows = np.concatenate([4 * (lanes >> 4)[:, None] + np.arange(4)[None, :],
                                   16 + 4 * (lanes >> 4)[:, None] + np.arange(4)[None, :]], axis=1)
            assert np.array_equal(got, (rows * 576 + col[:, None]).astype(np.uint16)), (w.wid, cb)


CODES, ROPE, SCALES = 0x10000000, 0x20000000, 0x30000000


@pytest.mark.parametrize("valid", [64, 37, 9, 1, 0])
def test_fp8_staging_and_dequant(fp8_mode, valid):
    """Staging loads stay inside their pages and LDS slot; after dequant every
    tile element is the exact widening of its own e4m3 code, rows past the
    valid count are zero, rope chunks are copied and scales land as [block][row]."""
    lds, tile, waves = {}, {}, []
    for w in range(4):
        m = Wave(w, lds)
        m.writes = tile
        m.run(lines_of(G.lane_constants) + lines_of(G.lane_constants_fp8))
        for k, v in ((G.S_PAGE, CODES), (G.S_PAGE + 1, 0), (G.S_RPAGE, ROPE), (G.S_RPAGE + 1, 0),
                     (G.S_SPAGE, SCALES), (G.S_SPAGE + 1, 0)):
            m.s[k] = v
        m.s[G.S_TMP + 21] = 1
        m.run(lines_of(G.dma_fp8, G.S_TMP + 21))
        for src, dst in m.loads:
            assert G.F8_RAW0 + G.F8_RAW <= dst and dst + 16 <= G.F8_RAW0 + 2 * G.F8_RAW
            base = CODES if src < ROPE else ROPE if src < SCALES else SCALES
            size = {CODES: G.F8_CODES, ROPE: G.F8_ROPE, SCALES: G.F8_SCALES}[base]
            assert 0 <= src - base and src - base + 16 <= size
        waves.append(m)
    for m in waves:
        m.s[G.S_SLOT], m.s[G.S_CURVALID] = 1, valid
        m.run(lines_of(G.dequant_fp8))
    for addr in tile:
        assert 0 <= addr < G.SLOT_BYTES or G.F8_SCL <= addr < G.F8_RF + 2048
    for r in range(64):
        for c in range(72):
            for q in range(4):
                got = tile.get(tile_byte(r, c) + 4 * q)
                if c < 64:
                    want = ("bf16", ("g", CODES + r * 512 + c * 8 + 2 * q), ("g", CODES + r * 512 + c * 8 + 2 * q + 1))
                    if r >= valid:
                        want = ("bf16", ZERO, ZERO)
                else:
                    want = tuple(("g", ROPE + r * 128 + (c - 64) * 16 + 4 * q + i) for i in range(4))
                    if r >= valid:
                        want = (ZERO,) * 4
                assert got == want, (r, c, q, got)
    for blk in range(4):
        for r in range(64):
            want = (ZERO,) * 4 if r >= valid else tuple(("g", SCALES + r * 16 + blk * 4 + i) for i in range(4))
            assert tile.get(G.F8_SCL + blk * 256 + r * 4) == want
    # reciprocal scales: rows r, r + 1 (r even) of block blk as bf16 pairs in the
    # 16 x 32 fragment of sub-step r / 32, in the probabilities' row order:
    # the hi pair at F8_RF + 1024 (r / 32) + 64 (4 blk) + 16 ((u % 16) / 4)
    # + 8 (u / 16) + 2 (u % 4), u = r % 32, the lo pair one fragment row (64 B)
    # on; the hi pair is formed from the two rows' own scales (zeroed past the
    # valid rows), the lo pair from the same scales and the hi pair
    for blk in range(4):
        for r in range(0, 64, 2):
            u = r % 32
            at = G.F8_RF + 1024 * (r // 32) + 256 * blk + 16 * ((u % 16) // 4) + 8 * (u // 16) + 2 * (u % 4)
            hi, lo = tile.get(at), tile.get(at + 64)
            assert hi is not None and lo is not None, (blk, r)
            assert hi[:2] == ("op", "v_cvt_pk_bf16_f32") and lo[:2] == ("op", "v_cvt_pk_bf16_f32")
            for k, row in enumerate((r, r + 1)):
                want = _leaves(("g", SCALES + row * 16 + blk * 4 + i) for i in range(4)) if row < valid \
                    else {ZERO}
                assert _leaves(hi[2 + k]) == want, (blk, row, hi)
                assert want <= _leaves(lo[2 + k]), (blk, row, lo)