"""Host-side checks of the decode kernels' LDS and global addressing.

The assembly generator's load, dequantize and read sequences are run lane by
lane by a small interpreter of the instructions they use, and the resulting
addresses are compared with the tile layout the kernels rely on: a tile slot
is 9 x 8 blocks of 1 KB; block (K, R) holds rows 8R..8R+7 and 16-byte chunks
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
                       "s_mov_b32": lambda: x[0]}[op]()

    def vector(self, op, a, L):
        V = lambda i: self.val(a[i], L)
        dst = lambda: int(re.fullmatch(r"v(\d+)", a[0]).group(1))
        arith = {"v_lshlrev_b32": lambda: V(2) << V(1), "v_lshrrev_b32": lambda: V(2) >> V(1),
                 "v_and_b32": lambda: V(1) & V(2), "v_xor_b32": lambda: V(1) ^ V(2),
                 "v_add_u32": lambda: V(1) + V(2), "v_mul_u32_u24": lambda: V(1) * V(2),
                 "v_lshl_add_u32": lambda: (V(1) << V(2)) + V(3), "v_lshl_or_b32": lambda: (V(1) << V(2)) | V(3),
                 "v_bfe_u32": lambda: (V(1) >> V(2)) & ((1 << V(3)) - 1), "v_mov_b32": lambda: V(1)}
        if op in arith:
            self.v[(dst(), L)] = arith[op]()
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
        elif op in ("ds_read_b64", "ds_read_b128", "ds_read_b64_tr_b16"):
            base, _, off = a[1].partition(" offset:")
            addr = self.val(base, L) + int(off or 0)
            self.reads.append((op, addr, L))
            if op != "ds_read_b64_tr_b16":
                n = 8 if op == "ds_read_b64" else 16
                d0 = int(re.match(r"v\[(\d+):", a[0]).group(1))
                byts = [self.lds.get(addr + b, ("undef",)) for b in range(n)]
                for q in range(n // 4):
                    self.v[(d0 + q, L)] = tuple(byts[4 * q:4 * q + 4])
        elif op in ("ds_write_b128", "ds_write_b32"):
            src, _, off = a[1].partition(" offset:")
            addr = self.val(a[0], L) + int(off or 0)
            if op == "ds_write_b32":
                self.writes[addr] = self.val(src, L)
            else:
                d0 = int(re.match(r"v\[(\d+):", src).group(1))
                for q in range(4):
                    self.writes[addr + 4 * q] = self.v[(d0 + q, L)]
        elif op == "global_load_lds_dwordx4":
            src = V(0) + self.sval(a[1])
            dst_addr = self.s["m0"] + 16 * L
            self.loads.append((src, dst_addr))
            for b in range(16):
                self.lds[dst_addr + b] = ("g", src + b)
        else:
            raise AssertionError(f"instruction not modelled: {op}")


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


@pytest.mark.parametrize("slot", [0, 1])
@pytest.mark.parametrize("valid", [64, 37, 8, 1])
def test_bf16_tile_loads(bf16_mode, slot, valid):
    """Each 16-byte tile chunk comes from its own row and chunk of the page
    (row 0 past the valid rows); each load moves eight whole 128-byte lines."""
    lds = {}
    for w in range(4):
        m = Wave(w, lds)
        m.run(lines_of(G.lane_constants))
        m.s[G.S_NVALID], m.s[G.S_TMP + 21] = valid, slot
        m.s[G.S_PAGE], m.s[G.S_PAGE + 1] = 0, 0
        m.run(lines_of(G.dma_setup, G.S_TMP + 21) + [i for g in G.dma_groups() for i in g])
        assert len(m.loads) == 18 * 64
        for k in range(18):
            lines = {src // 128 for src, _ in m.loads[64 * k:64 * k + 64]}
            if valid == 64:
                assert len(lines) == 8
    for r in range(64):
        for c in range(72):
            src = lds[slot * G.SLOT_BYTES + tile_byte(r, c)][1]
            row, rem = divmod(src, 1152)
            assert rem % 16 == 0 and 0 <= src and src + 16 <= 64 * 1152
            if r < valid:
                assert (row, rem // 16) == (r, c)
            else:
                assert row == 0 and rem // 16 // 8 == c // 8


def test_bf16_score_and_output_reads(bf16_mode):
    """Score reads: lane (g, r16) of fragment (ks, tb) reads row 32ss+16tb+r16,
    chunk 4ks+g.  Transposed output reads: lane (g, j) of column block cb reads
    row 32ss + 16 half + 4g + (j >> 2), columns 16cb + 4 (j & 3)."""
    m = Wave(0, {})
    m.run(lines_of(G.lane_constants))
    T = G.S_TMP
    for slot in (0, 1):
        m.s[T] = slot * G.SLOT_BYTES
        bases = [f"v_add_u32 v{G.V_UQ}, s{T}, v{G.V_QKE}", f"v_add_u32 v{G.V_UQ + 1}, s{T}, v{G.V_QKO}",
                 f"v_add_u32 v{G.V_UQ + 2}, 0x10000, v{G.V_UQ}", f"v_add_u32 v{G.V_UQ + 3}, 0x10000, v{G.V_UQ + 1}",
                 f"v_add_u32 v{G.V_UP}, s{T}, v{G.V_PV0}"]
        for k in range(1, 4):
            bases += [f"v_xor_b32 v{G.V_UP + k}, {32 * k}, v{G.V_PV0}", f"v_add_u32 v{G.V_UP + k}, s{T}, v{G.V_UP + k}"]
        m.run(bases)
        for ss in range(2):
            for i in range(36):
                m.reads = []
                m.run([x.format(buf="v[48:51]") for x in G.qk_read(ss, i)])
                ks, tb = divmod(i, 2)
                for op, addr, L in m.reads:
                    assert addr == slot * G.SLOT_BYTES + tile_byte(32 * ss + 16 * tb + (L & 15), 4 * ks + (L >> 4))
            for cb in range(32):
                m.reads = []
                m.run([x.format(lo="v[64:65]", hi="v[66:67]") for x in G.pv_read(ss, cb)])
                for n, (op, addr, L) in enumerate(m.reads):
                    half, g, j = n // 64, L >> 4, L & 15
                    row, col = 32 * ss + 16 * half + 4 * g + (j >> 2), 16 * cb + 4 * (j & 3)
                    assert addr == slot * G.SLOT_BYTES + tile_byte(row, col // 8) + (col % 8) * 2


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
        assert 0 <= addr < G.SLOT_BYTES or G.F8_SCL <= addr < G.F8_SCL + 1024
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
