"""Generate tile_h2.inc: the fixed-stabilizer tile work for waves that own
two 32-row halves of queries (64 rows), d = 128, as one inline-asm block.

Why asm: at two waves per SIMD a wave has 256 registers.  The output
accumulators of 64 rows x 128 channels take 128 of them (kept in AGPRs) and
the query fragments 64; hipcc cannot fit the rest of the tile in what is
left, so the tile work runs in fixed registers that this script schedules.

One 64-key tile (K and V^T tiles in LDS) is a chain of six parts; per 32-key
block kb:
  qk<kb>  scores S_h = K_kb Q_h^T for both halves h: 16 MFMAs, each K fragment
          read from LDS feeds both halves (the two chains alternate, which
          keeps every fragment read two pairs of products ahead with a ring
          of three);
  sm<kb>  weights x = fma(s, c, -mu_h); p = exp2(x); masked keys (tail,
          causal) get p = 0 under a branch on a uniform flag; the row sums
          l_h += p in fp32; p -> bf16 (round to nearest even) packed in place;
  pv<kb>  output O_h^T += V^T_kb P_h^T: 16 MFMAs, each V^T fragment read from
          LDS feeds both halves, and no VALU between them (a v_dot2 row sum
          there would hold the matrix pipeline: about 18 cycles each on
          gfx950).
The two waves of a SIMD run the chain half a tile apart: in the window
between two barriers the first wave runs pv1' qk0 sm0 pv0 qk1 sm1 and the
second sm1' pv1' qk0 sm0 pv0 qk1 (' = the previous tile's part), so that one
wave's weights, VALU only, overlap the other's products.  The block holds a
variant per case (a whole window, the first tile's, the drain after a wave's
last tile, loads only), chosen by the operand kind.  Each variant also issues
the wave's share of the next tile's loads into its LDS stage, spread between
the products.  The LDS layout and fragment addressing are those of
attn_bf16.hip (padded rows: fragment addresses are one base plus an
immediate).

Fixed registers: S_A = v[SB..SB+15], S_B = v[SB+16..SB+31] (scores, then
weights in place, then packed P in the first 8 of each), carried from one
window to the next as operands sc0/sc1; clobbered: the fragment ring F_j =
v[FB+4j..FB+4j+3], two address temporaries, s97 and m0.  Operands: O[h][c]
"+a" (16-AGPR tuples), l[h] "+v", q[h][s] "v" (4 VGPRs each), nm[h] "v"
(-mu), kad/vad "v" (per-lane fragment bases), ks/vs/vsp "s" (stage offsets of
the tile's K and V^T and of the previous tile's V^T), c2 "s", mf/mfp "s"
(mask flags of the tile and the previous one), lim[h] "v" (a weight of block
kb, register r is kept iff 32kb + 8(r/4) + (r%4) < lim[h]; the previous
tile's limits are 64 higher), kind "s"; for the loads rk/rv "s" (buffer
descriptors of the next K and V^T tiles), kdst/vdst "s" (their LDS
destinations), l4k/l16 "v" (per-lane sources), nld "s" (which loads).

Wait states are counted as hipcc counts them (one per instruction, N + 1 per
s_nop N): an MFMA result is read by VALU 12 later, a VALU result by an MFMA
5 later, a v_exp result by VALU 2 later; LDS reads are waited for with
lgkmcnt.  Each variant ends with enough s_nop for any MFMA still in flight:
afterwards the compiler may write its fixed registers or read the
accumulators.  The wave raises its priority (s_setprio) while it issues
products and lowers it for the weights: with two waves per SIMD, the one in
its weights phase then yields the issue slots to the other's products.

    python gen_tile_h2.py            # writes tile_h2.inc next to this file
"""
import os

D, NS, NC = 128, 8, 4
KSTR = D * 2 + 16          # LDS bytes per K row
VSTR = 64 * 2 + 16         # LDS bytes per V^T row
SB = 82                    # first score register
NF = 3                     # fragment ring slots
FB = SB + 32               # first fragment register
T0 = FB + 4 * NF           # address temporaries
PRIO = 3                   # wave priority while issuing MFMAs
ANCHOR_NOPS = 1            # no-ops after the block's 256-byte boundary
HZ_MFMA_VALU = 12
HZ_VALU_MFMA = 5
HZ_TRANS = 2
assert T0 + 1 == 127


class Gen:
    def __init__(self):
        self.out = []
        self.pos = 0
        self.ready_valu = {}   # vgpr -> first pos a VALU may read it
        self.ready_mfma = {}   # vgpr -> first pos an MFMA may read it
        self.pending = []      # outstanding LDS reads (fragment ids), issue order
        self.slot_of = {}
        self.slot_free = [True] * NF
        self.users_left = {}

    def emit(self, s, ws=1):
        self.out.append(s)
        self.pos += ws

    def pad(self, at):
        while self.pos < at:
            n = min(8, at - self.pos)
            self.emit(f"s_nop {n - 1}", n)

    # ---- LDS fragment reads
    def read(self, fid, text):
        j = self.slot_free.index(True)
        self.slot_free[j] = False
        self.slot_of[fid] = j
        self.emit(text.format(f=f"v[{FB + 4 * j}:{FB + 4 * j + 3}]"))
        self.pending.append(fid)

    def wait_frag(self, fid):
        if fid in self.pending:
            k = self.pending.index(fid)
            self.emit(f"s_waitcnt lgkmcnt({len(self.pending) - 1 - k})")
            del self.pending[:k + 1]

    def use_frag(self, fid):
        self.users_left[fid] -= 1
        if self.users_left[fid] == 0:
            self.slot_free[self.slot_of[fid]] = True

    # ---- instructions with hazard tracking
    def mfma(self, dst, a, b, c, reads_v):
        self.pad(max([self.ready_mfma.get(r, 0) for r in reads_v] + [0]))
        self.emit(f"v_mfma_f32_32x32x16_bf16 {dst}, {a}, {b}, {c}")
        return self.pos

    def valu(self, text, reads=(), writes=(), trans=False):
        self.pad(max([self.ready_valu.get(r, 0) for r in reads] + [0]))
        self.emit(text)
        for w in writes:
            self.ready_mfma[w] = self.pos + HZ_VALU_MFMA
            self.ready_valu[w] = self.pos + (HZ_TRANS if trans else 0)


def frag_k(kb, s, prev):
    return ("k", kb, s, prev)


def frag_v(kb, t, c, prev):
    return ("v", kb, t, c, prev)


NKR = 8      # key rows a wave loads per tile (64 rows, 8 waves)
NVC = 18     # 1 KB chunks of a V^T tile (128 rows of 144 bytes)


def load_items(tag):
    """The wave's share of the loads of the next tile into its LDS stage, one
    instruction list per load, issued between products so that the memory
    pipeline's queue never stalls the wave.  K: key rows 8w .. 8w + 7, one
    256-byte row a load (4 bytes a lane) into its padded LDS row; the load's
    immediate moves its LDS address too, hence M0 = row less 256 x j.  V^T:
    chunks w, w + 8 and (waves 0 and 1) w + 16 of the contiguous tile.  M0 is
    written by SALU one wait state before the load that reads it."""
    items = []
    for j in range(NKR):
        items.append([f"s_add_u32 m0, %[kdst], {j * (KSTR - 256)}", "s_nop 0",
                      f"buffer_load_dword %[l4k], %[rk], 0 offen offset:{j * 256} lds"])
    for j in range(3):
        so = "0" if j == 0 else "s97"
        ld = [f"s_add_u32 m0, %[vdst], {j * 8 * 1024}"]
        if j:
            ld.append(f"s_mov_b32 s97, {j * 8 * 1024}")
        else:
            ld.append("s_nop 0")
        ld.append(f"buffer_load_dwordx4 %[l16], %[rv], {so} offen lds")
        items.append(ld)
    # only while there is a next tile (%[nld] = its loads: 0 none, 2 all
    # chunks but the third V^T one, 3 all), and the third V^T chunk only
    # for the waves that have one
    for j, item in enumerate(items):
        label = f".Lnold{tag}{j}_%="
        need = 3 if j == NKR + 2 else 1
        assert NVC - 16 == 2
        items[j] = [f"s_cmp_lt_u32 %[nld], {need}", f"s_cbranch_scc1 {label}"] + item + [f"{label}:"]
    return items


def generate(parts, tag):
    """Instructions of the tile parts `parts`, a contiguous run of the chain
    ... qk0 sm0 pv0 qk1 sm1 pv1 qk0 ... of successive tiles, where a part
    name ending in "p" belongs to the previous tile (its V^T stage in operand
    vsp, its mask flag in mfp).  The current tile's stages are in ks/vs, its
    mask flag in mf, its per-half limits in lim0/lim1.  Fragment reads never
    cross the block's end: afterwards the fixed registers hold nothing but the
    scores / packed weights of the part in flight.  `tag` keeps labels apart."""
    ks, vs, vsp, mf, mfp, lim = "ks", "vs", "vsp", "mf", "mfp", "lim"
    g = Gen()
    last_phase = [None]
    loads = load_items(tag)
    n_mfma = sum(16 for p in parts if not p.startswith("sm"))
    every = max(1, n_mfma // (len(loads) + 1))
    count = [0]

    def after_mfma():
        count[0] += 1
        if loads and count[0] % every == 0:
            for line in loads.pop(0):
                g.emit(line, 0 if line.endswith(":") else 1)
    S = lambda h: SB + 16 * h
    g.emit("s_waitcnt lgkmcnt(0)")
    if any(p.startswith("qk") for p in parts):
        g.emit(f"v_add_u32 v{T0}, %[{ks}], %[kad]")
    vbase = [None]  # stage operand whose V^T base v[T0 + 1] holds
    # read stream in order of use
    stream = []
    for p in parts:
        kb, prev = int(p[2]), p.endswith("p")
        if p.startswith("qk"):
            for st in range(NS):
                stream.append((frag_k(kb, st, prev), f"ds_read_b128 {{f}}, v{T0} offset:{kb * 32 * KSTR + st * 32}",
                               None))
        elif p.startswith("pv"):
            for t in range(2):
                for c in range(NC):
                    stream.append((frag_v(kb, t, c, prev),
                                   f"ds_read_b128 {{f}}, v{T0 + 1} offset:{c * 32 * VSTR + (4 * kb + 2 * t) * 16}",
                                   vsp if prev else vs))
    for fid, _, _ in stream:
        g.users_left[fid] = 2
    nxt = [0]

    def refill():
        while nxt[0] < len(stream) and True in g.slot_free:
            fid, text, base = stream[nxt[0]]
            if base is not None and base != vbase[0]:
                # every read from the old base has been waited for: the
                # ring is shorter than the run of reads between two bases
                g.emit(f"v_add_u32 v{T0 + 1}, %[{base}], %[vad]")
                vbase[0] = base
            g.read(fid, text)
            nxt[0] += 1

    refill()
    valu_q = []  # VALU work waiting to be placed between MFMAs

    def drain_some(n):
        k = 0
        while valu_q and k < n:
            op = valu_q[0]
            if max([g.ready_valu.get(r, 0) for r in op[1]] + [0]) > g.pos:
                break  # not ready yet: the next MFMA first
            valu_q.pop(0)
            g.valu(*op)
            k += 1

    def weights(h):
        base = S(h)
        ops = []
        for r in range(16):
            ops.append((f"v_fma_f32 v{base + r}, v{base + r}, %[c2], %[nm{h}]", [base + r], [base + r]))
        for r in range(16):
            ops.append((f"v_exp_f32 v{base + r}, v{base + r}", [base + r], [base + r], True))
        return ops

    def mask(kb, h, prev):
        # the limits are those of the current tile; the previous tile's are
        # 64 keys higher
        base, flag, sh = S(h), (mfp if prev else mf), (-64 if prev else 0)
        label = f".Lnomask{tag}{kb}{h}{'p' if prev else ''}_%="
        body = [f"s_cmp_eq_u32 %[{flag}], 0", f"s_cbranch_scc1 {label}"]
        for r in range(16):
            body.append(f"v_cmp_lt_i32 vcc, {32 * kb + 8 * (r >> 2) + (r & 3) + sh}, %[{lim}{h}]")
            body.append(f"v_cndmask_b32 v{base + r}, 0, v{base + r}, vcc")
        body.append(f"{label}:")
        return body

    def packs(h):
        base = S(h)
        return [(f"v_cvt_pk_bf16_f32 v{base + e}, v{base + 2 * e}, v{base + 2 * e + 1}",
                 [base + 2 * e, base + 2 * e + 1], [base + e]) for e in range(8)]

    def sums(h):
        # l_h += the fp32 weights of the block (after masking, before the
        # bf16 packs), one dependent add each: the row sum is built in the
        # weights phase and the products phase carries no VALU (a v_dot2
        # would hold the matrix pipeline)
        base = S(h)
        return [(f"v_add_f32 %[l{h}], v{base + r}, %[l{h}]", [base + r], []) for r in range(16)]

    for p in parts:
        kb, prev = int(p[2]), p.endswith("p")
        # wave priority: high while issuing products, low during the weights,
        # so the other wave on the SIMD gets its products issued meanwhile
        g.emit(f"s_setprio {0 if p.startswith('sm') else PRIO}")
        # in the two main variants a weights phase starts once the fragment
        # reads already issued for the next products have landed (measured
        # faster together with the block's placement, see main())
        phase = "V" if p.startswith("sm") else "M"
        if tag in ("amain", "bmain") and last_phase[0] == "M" and phase == "V":
            g.emit("s_waitcnt lgkmcnt(0)")
        last_phase[0] = phase
        if p.startswith("qk"):
            # scores: the two halves' chains alternate, each K fragment feeds both
            for st in range(NS):
                fid = frag_k(kb, st, prev)
                g.wait_frag(fid)
                j = g.slot_of[fid]
                for h in range(2):
                    dst = f"v[{S(h)}:{S(h) + 15}]"
                    c = "0" if st == 0 else dst
                    # (st = 0: its result overwrites registers the row sums
                    # used; the wait covers that write after VALU writes)
                    q = g.mfma(dst, f"v[{FB + 4 * j}:{FB + 4 * j + 3}]", f"%[q{h}{st}]", c,
                               [FB + 4 * j + i for i in range(4)] + ([S(h) + r for r in range(16)] if st == 0 else []))
                    for r in range(16):
                        g.ready_valu[S(h) + r] = q + HZ_MFMA_VALU
                    g.use_frag(fid)
                    refill()
                    drain_some(2)
                    after_mfma()
        elif p.startswith("sm"):
            # weights in place, masks under the uniform flag, packs
            while valu_q:
                g.valu(*valu_q.pop(0))
            for h in range(2):
                for op in weights(h):
                    g.valu(*op)
                g.pad(max(g.ready_valu.get(S(h) + r, 0) for r in range(16)))
                for line in mask(kb, h, prev):
                    g.emit(line, 0 if line.endswith(":") else 1)
            for a, b in zip(sums(0), sums(1)):  # the halves' chains alternate
                g.valu(*a)
                g.valu(*b)
            for h in range(2):
                for op in packs(h):
                    g.valu(*op)
        else:
            # output products: each V^T fragment feeds both halves
            assert not valu_q
            for t in range(2):
                for c in range(NC):
                    fid = frag_v(kb, t, c, prev)
                    g.wait_frag(fid)
                    j = g.slot_of[fid]
                    for h in range(2):
                        pb = S(h) + 4 * t
                        g.mfma(f"%[o{h}{c}]", f"v[{FB + 4 * j}:{FB + 4 * j + 3}]", f"v[{pb}:{pb + 3}]",
                               f"%[o{h}{c}]", [FB + 4 * j + i for i in range(4)] + [pb + i for i in range(4)])
                        g.use_frag(fid)
                        refill()
                        after_mfma()
            while valu_q:
                g.valu(*valu_q.pop(0))
    for item in loads:  # what did not fit between products
        for line in item:
            g.emit(line, 0 if line.endswith(":") else 1)
    assert not g.pending and nxt[0] == len(stream)
    g.emit("s_setprio 0")
    # The fixed registers are free to the compiler once the block ends, while
    # the last products may still be reading their operands from them (and
    # writing the accumulators): wait out an MFMA before leaving.
    g.emit("s_nop 7")
    g.emit("s_nop 7")
    g.emit("s_nop 3")
    return g.out


# The window of one tile: the waves of a SIMD's pair run the chain half a tile
# apart, so that one's weights overlap the other's products.  Variant ids
# are those of the kernel's `kind` operand.
VARIANTS = [
    ("amain", ["pv1p", "qk0", "sm0", "pv0", "qk1", "sm1"]),   # 0: first wave of the pair
    ("bmain", ["sm1p", "pv1p", "qk0", "sm0", "pv0", "qk1"]),  # 1: second wave
    ("afirst", ["qk0", "sm0", "pv0", "qk1", "sm1"]),          # 2: first tile
    ("bfirst", ["qk0", "sm0", "pv0", "qk1"]),                 # 3
    ("adrain", ["pv1p"]),                                      # 4: after the last tile
    ("bdrain", ["sm1p", "pv1p"]),                              # 5
    ("loads", []),                                             # 6: only the loads
]


def main():
    here = os.path.dirname(os.path.abspath(__file__))
    text = ["// tile_h2.inc -- generated by gen_tile_h2.py; do not edit.",
            "// Fixed-stabilizer tile window, two 32-row query halves per wave, d = 128."]
    # Placement.  The block's performance depends on where its instructions
    # sit relative to 256-byte boundaries (layouts that differ by a few
    # no-ops measured up to 7% apart), so it starts at a fixed offset from
    # one: a jump over padding to a 256-byte boundary, then ANCHOR_NOPS
    # no-ops (the best of the offsets measured), and its end is padded to a
    # 64-byte boundary, so the code around it does not move it and it does
    # not move the code after it by less than that.
    lines = ["s_branch .Lanchor_%=", ".p2align 8", ".Lanchor_%=:"] + ["s_nop 0"] * ANCHOR_NOPS
    for i, (tag, _) in enumerate(VARIANTS[1:], 1):
        lines += [f"s_cmp_eq_u32 %[kind], {i}", f"s_cbranch_scc1 .Lv{tag}_%="]
    for i, (tag, parts) in enumerate(VARIANTS):
        body = generate(parts, tag)
        n_mfma = sum(1 for l in body if "mfma" in l)
        n_rd = sum(1 for l in body if l.startswith("ds_read"))
        text.append(f"// {i} {tag}: {' '.join(parts)}: {n_mfma} MFMAs, {n_rd} LDS fragment reads, "
                    f"{len(body)} instructions")
        print(f"{tag}: {len(body)} instructions, {n_mfma} MFMAs")
        if i > 0:
            lines.append(f".Lv{tag}_%=:")
        lines += body
        lines.append("s_branch .Lend_%=")
    lines[-1] = ".p2align 6"
    lines.append(".Lend_%=:")
    body = " \\\n".join(f'  "{l}\\n"' for l in lines)
    text.append(f"#define CLIS_TILE_H2_WINDOW \\\n{body}")
    text.append("#define CLIS_TILE_H2_CLOBBERS \\")
    text.append("  " + ", ".join(f'"v{r}"' for r in range(FB, T0 + 2)) + ', "s97", "m0", "vcc", "scc", "memory"')
    with open(os.path.join(here, "tile_h2.inc"), "w") as f:
        f.write("\n".join(text) + "\n")


if __name__ == "__main__":
    main()
