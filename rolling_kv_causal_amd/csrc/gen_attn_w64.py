"""Writes attn_w64_asm.h: the tile loop of the 64-row attention kernel as one asm program.

Run from this directory (`python3 gen_attn_w64.py > attn_w64_asm.h`); the header is committed
and a host test checks that it matches this script's output.

One wave owns 64 query rows (two 32-row blocks qb) of one (element, head).  Per 64-key tile it
issues 64 MFMAs 32x32x16 bf16 fed by 32 LDS fragment reads (each read feeds both row blocks):
  QK:  S^T[kb][qb] = K[kb] Q^T[qb]      16 K reads (kb-major, 8 k steps each)
  PV:  O^T[db][qb] += V^T[db] P^T[qb]   16 V^T reads (key step ks-major, d block db)
and, interleaved with the MFMAs from the 20th on (S^T of key block 0 is complete after the
16th), the softmax of the tile's S into bf16 P^T words for the next tile's PV: Q^T holds the
stored bf16 queries unchanged and the first QK MFMA of a chain accumulates onto the
-(m + BIAS) / scale_log2 block, so scale_log2 * S (one fp32 product per score) is the exponent;
the P words are ORed for the lazy test, and eight 16x16x32 MFMAs add the previous tile's P row
sums into l.  Three programs: SDV2_W64_LOOP as described; SDV2_W64_LOOP_SK for a bf16 cache
whose keys carry scale_log2 (the host passes scale_log2 = 1 and the exponentials read S
directly: no product); SDV2_W64_LOOP_FP8 for the e4m3 cache, which carries it too (with the
queries staged times a power of two), and differs from SK only in its loads: staged by one
iteration, widened to bf16 in the first gaps of the next one.

Iteration t, t mod 4 = phase ph (every state register is an asm operand, so the compiler never
moves them; the loop is generated once per phase, so the ring slots of K(t) (ph) and V^T(t-1)
(ph - 1) are immediate offsets of the fragment reads):
  bf16: wait for the loads of iteration t-2; barrier (e4m3: every wave has written its share of
    K(t), V^T(t-1), widened in iteration t-1); branch on mflag(t) to the masked variant
  tile block: QK(t), PV(t-1) with P buffer pp, softmax(t) into buffer 1-pp, this wave's tile
    loads (K(t+2), V^T(t+1); bf16 eight of 1 KB into the ring, e4m3 four into the staging
    slot of parity ph mod 2) spread over the stream, e4m3: the widening of this wave's staged
    K(t+1), V^T(t) (loaded in iteration t-1) into ring slots ph + 1 and ph in the gaps before the
    softmax, in the registers of the P buffer it is about to fill, and, in the free issue slots of the QK
    part, the scalar set-up of iteration t+1 (load cursors and global bases, the walk cursor
    and mflag of tile t+1); then the lazy test (trig != 0: some P word of the tile is >= 2 or
    not finite, or some row has no maximum yet)
  trig != 0 (out of line): the rescale: masked row max, m, alpha, O and l scaled (not while
    no row of the block has a maximum), P of the tile recomputed into buffer 1-pp, the -m
    blocks rewritten
After the loop the last PV.  (e4m3: before the loop, K(0) and the zeroed V^T(-1) are widened.)  Set-up values alternate between
two register sets by iteration parity, so the loads of iteration t read one set while the
stream writes the other.  The masked variant ANDs every P word with its mask word: the
ragged-tile mask (keys >= nvalid) times the row block's causal mask (own frame tk after the
row's frame), computed at the block start into AGPRs.

Register plan (per lane):
  a[0:127]    O^T  o[db][qb] at a[(2db+qb)*16 .. +15]
  a[128:191]  Q^T  q[qb][kd] at a[128 + (8qb+kd)*4 .. +3]
  v[0:63]     S^T  s[kb][qb] at v[(2kb+qb)*16 .. +15]
  v[64:127]   P^T  two buffers, p[qb][ks] at base + (4qb+ks)*4, base 64 or 96
  v[128:175]  fragment ring, 12 slots of 4 (also rare-path temporaries)
  v[176:183]  K fragment LDS addresses per k step kd;  v[184:187] V^T addresses per key step
  v[188:199]  temporaries
  v[200:201]  m per qb (running max, log2 units)
  v[202:233]  -(m + BIAS) / scale_log2 blocks per qb (first QK accumulator)
  v[236:243]  K and V^T lane offsets of the tile loads;  v244 frame slots
  v245        mask temporary;  v246 OR of the tile's P words
  v[248:255]  l accumulators (16x16 MFMA layout), four per qb
  a[192:223]  mask words per (qb, word);  a[224:227] 8g, frame per qb, (lane ^ 32) * 4
  a[228:231]  row-sum selector
  e4m3 only:  v[234:235] staging read addresses; a[232:239] widened-chunk write addresses
              (read into v[188:195] for the widening)
  s[84:91]    global bases of the K and V^T tile loads, two sets by iteration parity

Hazards kept by construction (gfx950, counted in issued instructions): an MFMA result is read
by no VALU or MFMA A/B operand within 12 instructions (checked below; the rare block starts
with 16 wait states); VALU-written P words are read by MFMAs of the next tile only; an
exponential's result is read at least one instruction later; a register an MFMA reads is not
overwritten by an LDS read or a VALU op within 12 instructions (an MFMA may read its A operand
after issue, so 8 reads in flight use a ring of 12 slots); an LDS DMA load does not directly
follow a write of m0; same-accumulator MFMAs chain back to back (allowed); VOP3 forms read at
most one SGPR; a VALU-written SGPR (readlane) is read by the scalar unit only after the next
MFMA (measured: the wave stalls about 20 cycles otherwise).  Measured on gfx950 and avoided: a dot2 (v_dot2_f32_bf16) waits for the MFMA in flight
to finish, and its result is not interlocked for a non-dot2 reader (3 wait states needed).
"""
import sys

KA = 8                                           # fragment reads in flight
RING = 12                                        # fragment slots: a slot is refilled 4 reads after its last use
FR, KADDR, VADDR = 128, 176, 184
TMP, M = 188, 200
TS = 248                                         # l accumulators, four per row block (16x16 MFMA layout)
NEG_INF = "0xff800000"
SM_FROM = 20                                     # first MFMA followed by softmax VALU ops
WAIT_EVERY = 4                                   # one LDS wait per this many fragment reads
READ_START = 2                                   # fragment reads issued before the first MFMA
NEXT_GAP = ["<next gap>"]                        # unit marker: continue the chunk after the next MFMA
LATE = "<late>"                                  # widen unit marker: issue after its MFMA pair's fragment reads
GAP_CAP = 5                                      # instructions between two MFMAs the set-up may fill up to
WIDEN_CAP = 8                                    # ... and the e4m3 widening (set-up included)
WIDEN_END = 16                                   # e4m3: first gap of the set-up, after most of the widening


def o_reg(db, qb):
    b = (db * 2 + qb) * 16
    return f"a[{b}:{b + 15}]"


def o_elem(db, qb, v):
    return f"a{(db * 2 + qb) * 16 + v}"


def q_reg(qb, kd):
    b = 128 + (qb * 8 + kd) * 4
    return f"a[{b}:{b + 3}]"


def s_reg(kb, qb):
    b = (kb * 2 + qb) * 16
    return f"v[{b}:{b + 15}]"


def s_elem(kb, qb, v):
    return f"v{(kb * 2 + qb) * 16 + v}"


def rowsum_mfma(pp, qb, ks):
    """bf16: l += row sums of P^T[qb][ks] (16 keys) on the matrix core.  Read as the B operand
    of a 16x16x32 MFMA, lane (g, r) of the P^T quad is column r mod 16 and k-block 2g + r / 16;
    the selector (ones at lanes 0 and 32 for output row 0, 17 and 49 for row 1) sums row r < 16
    into output row 0 and row r >= 16 into output row 1 of column r mod 16: lane j < 16 holds
    l(row j) in its first and l(row j + 16) in its second accumulator register."""
    b = TS + 4 * qb
    return f"v_mfma_f32_16x16x32_bf16 v[{b}:{b + 3}], a[{SEL}:{SEL + 3}], {p_reg(pp, qb, ks)}, v[{b}:{b + 3}]"


def cb_reg(qb):
    b = CB + 16 * qb
    return f"v[{b}:{b + 15}]"


def p_base(buf):
    return 64 if buf == 0 else 96


def p_reg(buf, qb, ks):
    b = p_base(buf) + (qb * 4 + ks) * 4
    return f"v[{b}:{b + 3}]"


def p_word(buf, qb, ks, w):
    return f"v{p_base(buf) + (qb * 4 + ks) * 4 + w}"


def frag(slot):
    b = FR + slot * 4
    return f"v[{b}:{b + 3}]"


def word_key(j):
    """Key offset (without 8g) of the low half of P word j = 4 ks + w of a row block."""
    return 32 * (j >> 3) + 16 * ((j >> 2) & 1) + 2 * (j & 3)


def k_reads():
    # kb-major: S^T of key block 0 is complete after the first 16 MFMAs, so the softmax of its
    # half of the tile overlaps the key block 1 MFMAs
    return [("K", kb, kd) for kb in range(2) for kd in range(8)]


def v_reads():
    return [("V", db, ks) for ks in range(4) for db in range(4)]


def read_instr(r, slot, ph):
    """LDS read of fragment r in iteration phase ph (t mod NSLOT): K(t) sits in ring slot
    ph, V^T(t-1) in slot ph - 1; the slot is the instruction's offset."""
    if r[0] == "K":
        _, kb, kd = r
        return f"ds_read_b128 {frag(slot)}, v{KADDR + kd} offset:{(ph % NSLOT) * KTILE + kb * 8192}"
    _, db, ks = r
    return f"ds_read_b128 {frag(slot)}, v{VADDR + ks} offset:{((ph - 1) % NSLOT) * KTILE + db * 4096}"


def mfma_pair(r, slot, pp):
    out = []
    if r[0] == "K":
        _, kb, kd = r
        for qb in range(2):
            c = s_reg(kb, qb) if kd else cb_reg(qb)
            out.append(f"v_mfma_f32_32x32x16_bf16 {s_reg(kb, qb)}, {frag(slot)}, {q_reg(qb, kd)}, {c}")
    else:
        _, db, ks = r
        for qb in range(2):
            out.append(f"v_mfma_f32_32x32x16_bf16 {o_reg(db, qb)}, {frag(slot)}, {p_reg(pp, qb, ks)}, {o_reg(db, qb)}")
    return out


def softmax_ops(pc, masked, qbs=(0, 1), mreg=None):
    """Groups of 4 values of S (s - (m + BIAS) / scale_log2, in the units of the stored q and
    k): 4 products by scale_log2 in fp32, 4 exponentials, 2 packs into P words and, in the
    tile's stream, an OR of the words into the lazy-test accumulator.  Masked, every P word is
    ANDed with its mask word (ragged tile and causal), so masked keys weigh and sum to nothing.
    mreg(qb): given only when the rescale recomputes P, the register holding the shift
    subtracted after the product (one fma).  (The row sums run on the matrix core.)
    SCALED (keys cached times scale_log2, which the host then passes as 1): S is already the
    exponent, so the exponentials read the accumulator and there is no product."""
    shifted = mreg is not None
    ops = []
    gi = 0
    for kb in range(2):
        for qb in qbs:
            for half in range(2):
                ks = 2 * kb + half
                for w0 in (0, 2):
                    t = [f"v{TMP + (gi % 3) * 4 + j}" for j in range(4)]
                    gi += 1
                    vs = [half * 8 + 2 * w0 + j for j in range(4)]
                    if shifted:            # S * scale_log2 - shift
                        for j in range(4):
                            ops.append(f"v_fma_f32 {t[j]}, {s_elem(kb, qb, vs[j])}, %[sl], -{mreg(qb)}")
                        src = t
                    elif SCALED:           # S = s - m - BIAS already
                        src = [s_elem(kb, qb, vs[j]) for j in range(4)]
                    else:                  # S * scale_log2 = s * scale_log2 - m - BIAS
                        for j in range(4):
                            ops.append(f"v_mul_f32 {t[j]}, %[sl], {s_elem(kb, qb, vs[j])}")
                        src = t
                    for j in range(4):
                        ops.append(f"v_exp_f32 {t[j]}, {src[j]}")
                    words = [p_word(pc, qb, ks, w0), p_word(pc, qb, ks, w0 + 1)]
                    ops.append(f"v_cvt_pk_bf16_f32 {words[0]}, {t[0]}, {t[1]}")
                    ops.append(f"v_cvt_pk_bf16_f32 {words[1]}, {t[2]}, {t[3]}")
                    if masked:
                        for wi, w in enumerate(words):
                            j = ks * 4 + w0 + wi
                            ops.append(f"v_accvgpr_read_b32 v{MT}, a{MKA + 16 * qb + j}")
                            ops.append(f"v_and_b32 {w}, {w}, v{MT}")
                    if not shifted:            # the lazy test of the tile: OR of its P words
                        ops.append(f"v_or_b32 v{ACC}, {words[0]}, {words[1]}" if gi == 1 else
                                   f"v_or3_b32 v{ACC}, v{ACC}, {words[0]}, {words[1]}")
    return ops


def mask_setup():
    """Ragged masks: low half of word j valid iff 8g + key(j) < nvalid, high half iff
    8g + key(j) + 1 < nvalid.  Causal mask of qb: all ones iff tk <= frame of the row.
    The product of both per (qb, word) goes to a[192 + 16 qb + j]."""
    g8, tq0, tq1 = (f"v{TMP + 5}", f"v{TMP + 6}", f"v{TMP + 7}")
    lines = [f"v_accvgpr_read_b32 {g8}, a{LANEA}", f"v_accvgpr_read_b32 {tq0}, a{LANEA + 1}",
             f"v_accvgpr_read_b32 {tq1}, a{LANEA + 2}",
             f"v_mov_b32 v{TMP + 2}, 0xffff", f"v_mov_b32 v{TMP + 3}, 0xffff0000", f"v_mov_b32 v{TMP + 4}, -1"]
    for qb in range(2):
        lines += [f"v_cmp_le_i32 vcc, %[tk], v{TMP + 6 + qb}",
                  f"v_cndmask_b32 v{TMP + 8 + qb}, 0, v{TMP + 4}, vcc"]
    for j in range(16):
        c = word_key(j)
        lines += [f"s_sub_i32 %[stmp], %[nvalid], {c}",
                  f"v_cmp_gt_i32 vcc, %[stmp], {g8}",
                  f"v_cndmask_b32 v{TMP}, 0, v{TMP + 2}, vcc",
                  f"s_sub_i32 %[stmp], %[nvalid], {c + 1}",
                  f"v_cmp_gt_i32 vcc, %[stmp], {g8}",
                  f"v_cndmask_b32 v{TMP + 1}, 0, v{TMP + 3}, vcc",
                  f"v_or_b32 v{TMP + 10}, v{TMP}, v{TMP + 1}"]
        for qb in range(2):
            lines += [f"v_and_b32 v{TMP + 11}, v{TMP + 10}, v{TMP + 8 + qb}",
                      f"v_accvgpr_write_b32 a{MKA + 16 * qb + j}, v{TMP + 11}"]
    return lines


def stream(reads, pp, ph, valu, dma=None, valu_from=0, extra=(), widen=()):
    """Reads KA ahead of their MFMAs (after a ramp: READ_START reads before the first MFMA, then
    two per MFMA pair until KA are in flight); VALU ops spread evenly over the MFMAs from index
    valu_from on.  dma maps a read index i to (m0 setup, tile load): the setup follows the MFMA
    pair of read i and the load the LDS read issued after it, so the tile loads of a wave are
    spread over the tile instead of queueing behind the other waves' loads at the texture unit.
    extra: (first gap, units) chunks of scalar bookkeeping, placed in order and one chunk after
    the other; a unit (a few instructions, closed in its use of SCC) goes into the gap after an
    MFMA, from the chunk's first gap on, into the first gap with room for it (at most GAP_CAP
    instructions besides the MFMA), so the wave can issue it while the matrix core works.
    widen: (first gap, unit) pairs (e4m3), placed in order after the set-up, each from its first
    gap on into the first gap with room (WIDEN_CAP), all before the softmax's first gap; a unit
    that starts with LATE goes, on a cursor of its own, after the fragment reads that follow the
    MFMA pair of its first gap, one such unit per pair.  Waits
    are written as marks and resolved at the end: lgkmcnt(@Fi) waits for fragment read i and
    lgkmcnt(@Wj) for widening read j, counting every LDS op issued after it (LDS ops complete in
    order); vmcnt(@Pj) waits for load j of the previous iteration's four (e4m3), counting the
    loads this stream has issued since."""
    dma = dma or {}
    out = []                                     # (line, tag): tags name the reads waited for
    # reads issued after the MFMA pair of read i: KA ahead in the steady state; the stream starts
    # with READ_START reads and catches up by one extra read per pair, so the four waves leaving
    # the barrier together do not queue 32 reads at the LDS at once
    first = min(READ_START, len(reads))
    after = []
    nr = first
    for i in range(len(reads)):
        upto = min(len(reads), i + KA + 1, nr + 2)
        after.append(list(range(nr, upto)))
        nr = upto
    assert nr == len(reads)
    for i in range(first):
        out.append((read_instr(reads[i], i % RING, ph), f"F{i}"))
    # LDS waits: before the MFMA pair of read i when read i is not yet covered; a wait covers
    # reads up to i + WAIT_EVERY - 1, but not those issued after the previous pair (during the
    # ramp they would stall the wave), and at least read i.  waits[i] = last read covered.
    waits, done, n_issued = {}, 0, first
    for i in range(len(reads)):
        if i >= done:
            recent = len(after[i - 1]) if i else 0
            done = max(i + 1, min(i + WAIT_EVERY, n_issued - recent))
            # (at most 15 reads may stay in flight)
            waits[i] = max(done, n_issued - 15) - 1
        n_issued += len(after[i])
    n_mfma = 2 * len(reads)
    fixed = [0] * n_mfma                         # read, wait and load instructions after MFMA g
    for i in range(len(reads)):
        fixed[2 * i + 1] += (i + 1 in waits) + len(after[i]) + 2 * (i in dma)
    # VALU ops in order over the gaps from valu_from on, levelling VALU + fixed per gap
    per = [0] * n_mfma
    region = range(valu_from, n_mfma)
    level = (len(valu) + sum(fixed[g] for g in region)) / len(region)
    vi, done, goal = 0, 0, 0.0
    for g in region:
        goal += level
        while vi < len(valu) and done + fixed[g] + per[g] + 1 <= goal + 0.5:
            per[g] += 1
            vi += 1
        done += fixed[g] + per[g]
    per[n_mfma - 1] += len(valu) - vi
    load = [per[g] + fixed[g] for g in range(n_mfma)]
    placed = [[] for _ in range(n_mfma)]
    g = 0
    for first_gap, units in extra:
        # chunks one after another: they share the scratch SGPRs x and y
        g = max(g, first_gap)
        for u in units:
            if u == NEXT_GAP:                    # the rest of the chunk goes after the next MFMA
                g = min(g + 1, n_mfma - 1)
                continue
            while g < n_mfma - 1 and load[g] + len(u) > GAP_CAP:
                g += 1
            placed[g] += u
            load[g] += len(u)
    wplaced = [[] for _ in range(n_mfma)]
    late = [[] for _ in range(len(reads))]       # issued after the fragment reads of MFMA pair i
    g, gl = 0, 0
    for first_gap, u in widen:
        if u and u[0] == LATE:
            gl = max(gl, first_gap)
            while late[gl // 2]:
                gl += 2
            assert gl < valu_from, "the widening must end before the softmax reuses its registers"
            late[gl // 2] += u[1:]
            load[gl | 1] += len(u) - 1
            continue
        g = max(g, first_gap)
        while g < valu_from and load[g] + len(u) > WIDEN_CAP:
            g += 1
        assert g < valu_from, "the widening must end before the softmax reuses its registers"
        wplaced[g] += u
        load[g] += len(u)
    vi = 0
    for i, r in enumerate(reads):
        if i in waits:
            out.append((f"s_waitcnt lgkmcnt(@F{waits[i]})", None))
        for j, m in enumerate(mfma_pair(r, i % RING, pp)):
            out.append((m, None))
            for _ in range(per[2 * i + j]):
                out.append((valu[vi], None))
                vi += 1
            out += [(x, None) for x in placed[2 * i + j]]
            out += [(x, None) if isinstance(x, str) else x for x in wplaced[2 * i + j]]
        if i in dma:
            out.append((dma[i][0], None))
        for j in after[i]:
            out.append((read_instr(reads[j], j % RING, ph), f"F{j}"))
        if i in dma and not after[i]:
            out.append(("s_nop 0", None))
        if i in dma:
            out.append((dma[i][1], None))
        out += [(x, None) for x in late[i]]
    assert vi == len(valu)
    out.append(("s_waitcnt lgkmcnt(0)", None))
    return resolve_waits(out)


def resolve_waits(out):
    """Lines with their wait marks replaced: lgkmcnt(@tag) by the number of LDS ops issued after
    the tagged one (at most 15: waiting for more is safe), vmcnt(@Pj) by 3 - j plus the tile
    loads issued since the stream began."""
    lines, lds, loads = [], [], 0
    for text, tag in out:
        op = text.split()[0]
        if "lgkmcnt(@" in text:
            want = text.split("(@")[1].rstrip(")")
            n = len(lds) - 1 - lds.index(want)
            text = f"s_waitcnt lgkmcnt({min(n, 15)})"
        elif "vmcnt(@P" in text:
            j = int(text.split("(@P")[1].rstrip(")"))
            text = f"s_waitcnt vmcnt({3 - j + loads})"
        if op.startswith("ds_"):
            lds.append(tag)
        if op.startswith("global_load"):
            loads += 1
        lines.append(text)
    return lines


def tile_block(ph, masked):
    """Iteration phase ph (t mod NSLOT; parity par = ph mod 2, P buffer pp = 1 - par):
    QK(t), PV(t-1) with P buffer pp, softmax(t) into buffer 1-pp, this iteration's tile loads
    (bases of parity par) and the next iteration's scalar set-up, then the lazy test
    (trig != 0: some P word of the tile is >= 2 or not finite, or a row has no maximum yet)."""
    par = ph % 2
    pp = 1 - par
    pc = 1 - pp
    lines = mask_setup() if masked else []
    # (e4m3: after the widening, which takes the first gaps)
    g0 = WIDEN_END if F8 else 0
    extra = [(g0, v_setup(1 - par)), (g0, cursor_shift()), (g0, k_setup(1 - par, 3)),
             (g0, walk_setup(1 - par, False))]
    valu = softmax_ops(pc, masked)
    # l += row sums of P(t-1) (buffer pp, complete), one MFMA after every other group
    sums = [rowsum_mfma(pp, qb, ks) for ks in range(4) for qb in range(2)]
    out, gcount = [], 0
    for op in valu:
        out.append(op)
        if op.startswith(("v_or_b32", "v_or3_b32")) and f"v{ACC}" in op:
            gcount += 1
            if gcount % 2 == 1 and sums:
                out.append(sums.pop(0))
    valu = out + sums
    lines += stream(k_reads() + v_reads(), pp, ph, valu, tile_loads(ph), SM_FROM, extra,
                    widen_units(ph, pc) if F8 else ())
    # lazy test: some P word >= 2 (a score 9 above m, or not finite), or a row without m
    return lines + [f"v_and_b32 v{TMP}, 0x40004000, v{ACC}",
                    f"v_cmp_ne_u32 vcc, 0, v{TMP}",
                    "s_mov_b64 %[trig], vcc",
                    "s_or_b64 %[trig], %[trig], %[ninf]"]


RARE_ID = [0]                                    # unique labels of the rare blocks


def rare_block(pc, masked):
    """Rescale of the tile: S = s - (mc + BIAS) / scale_log2, mc = m if finite, else 0.  New row
    maximum m' = max(m, scale_log2 * (max over valid keys of S) + mc + BIAS); O, l scaled by
    2^(m - m') (not while no row of the block has a maximum: both are zero then); the tile's P
    recomputed as 2^(S scale_log2 - (mc' - mc)) with mc' = m' if finite, else 0; the -m block of
    the row block set to -(mc' + BIAS) / scale_log2; ninf: lanes whose row still has m = -inf."""
    mx, y, mn, al, mcn, t0, t1, ninf = (f"v{x}" for x in range(128, 136))
    mc, dd, bp = "v144", "v145", "v146"
    lines = ["s_nop 15", f"v_mov_b32 {ninf}, {NEG_INF}", f"v_accvgpr_read_b32 {bp}, a{LANEA + 3}"]
    for qb in range(2):
        lines.append(f"v_mov_b32 {mx}, {NEG_INF}")
        for j in range(16):
            kb, v = j >> 3, ((j >> 2) & 1) * 8 + 2 * (j & 3)
            lo, hi = s_elem(kb, qb, v), s_elem(kb, qb, v + 1)
            if masked:
                lines += [f"v_accvgpr_read_b32 {t0}, a{MKA + 16 * qb + j}",
                          f"v_and_b32 {t1}, 0xffff, {t0}",
                          f"v_cmp_ne_u32 vcc, 0, {t1}",
                          f"v_cndmask_b32 {t1}, {ninf}, {lo}, vcc",
                          f"v_max_f32 {mx}, {mx}, {t1}",
                          f"v_cmp_lt_u32 vcc, 0xffff, {t0}",
                          f"v_cndmask_b32 {t1}, {ninf}, {hi}, vcc",
                          f"v_max_f32 {mx}, {mx}, {t1}"]
            else:
                lines.append(f"v_max3_f32 {mx}, {mx}, {lo}, {hi}")
        lines += [f"ds_bpermute_b32 {y}, {bp}, {mx}",
                  "s_waitcnt lgkmcnt(0)",
                  f"v_max_f32 {mx}, {mx}, {y}",
                  f"v_mul_f32 {mx}, %[sl], {mx}",                      # scale_log2 > 0 keeps the max
                  f"v_cmp_eq_f32 vcc, {NEG_INF}, v{M + qb}",
                  f"v_cndmask_b32_e64 {mc}, v{M + qb}, 0, vcc",       # mc: m, 0 while m = -inf
                  "s_cmp_eq_u64 vcc, exec",                            # no row has a maximum yet:
                  f"v_add_f32 {t0}, {mx}, {mc}",
                  f"v_add_f32 {t0}, {hex(0x41000000)}, {t0}",                  # + BIAS (8.0)
                  f"v_max_f32 {mn}, v{M + qb}, {t0}",                 # m'
                  f"v_sub_f32 {t0}, v{M + qb}, {mn}",
                  f"v_exp_f32 {al}, {t0}",
                  f"v_cmp_eq_f32 vcc, {NEG_INF}, {mn}",
                  f"v_cndmask_b32_e64 {al}, {al}, 1.0, vcc",          # alpha = 1 if m' = -inf
                  f"v_cndmask_b32_e64 {mcn}, {mn}, 0, vcc",           # mc'
                  f"v_sub_f32 {dd}, {mcn}, {mc}",
                  f"v_mov_b32 v{M + qb}, {mn}",
                  f"s_cbranch_scc1 .Lw64_ns{RARE_ID[0]}_%=",         # O and l are 0: no scaling
                  # l of row j (< 16) sits in lane j, register 0; of row j + 16 in lane j, register 1
                  f"v_mul_f32 v{TS + 4 * qb}, v{TS + 4 * qb}, {al}",
                  f"v_xor_b32 {t1}, 0xc0, {bp}",                       # (lane ^ 16) * 4
                  f"ds_bpermute_b32 {y}, {t1}, {al}",
                  "s_waitcnt lgkmcnt(0)",
                  f"v_mul_f32 v{TS + 4 * qb + 1}, v{TS + 4 * qb + 1}, {y}"]
        vals = [(db, v) for db in range(4) for v in range(16)]
        for k in range(0, 64, 4):
            grp = vals[k:k + 4]
            tmps = [f"v{136 + i}" for i in range(4)]   # v136..v139
            lines += [f"v_accvgpr_read_b32 {tmps[i]}, {o_elem(db, qb, v)}" for i, (db, v) in enumerate(grp)]
            lines += [f"v_mul_f32 {tmps[i]}, {tmps[i]}, {al}" for i in range(4)]
            lines += [f"v_accvgpr_write_b32 {o_elem(db, qb, v)}, {tmps[i]}" for i, (db, v) in enumerate(grp)]
        lines.append(f".Lw64_ns{RARE_ID[0]}_%=:")
        RARE_ID[0] += 1
        lines += softmax_ops(pc, masked, qbs=(qb,), mreg=lambda _q: dd)
        lines.append(f"v_sub_f32 {t0}, {hex(0xc1000000)}, {mcn}")                  # -(mc' + BIAS)
        lines.append(f"v_mul_f32 {t0}, %[slinv], {t0}")                            # / scale_log2
        lines += [f"v_mov_b32 v{CB + 16 * qb + i}, {t0}" for i in range(16)]
    lines += [f"v_cmp_eq_f32 vcc, {NEG_INF}, v{M}", "s_mov_b64 %[ninf], vcc",
              f"v_cmp_eq_f32 vcc, {NEG_INF}, v{M + 1}", "s_or_b64 %[ninf], %[ninf], vcc"]
    return lines


def init_block():
    """O = 0 and P(-1) = 0 (read by the first PV), written sixteen registers at a time by MFMAs
    of zero operands; m = -inf; the -m blocks -BIAS / scale_log2 (nbias), the row-sum
    accumulators 0, every row flagged."""
    zero = "v[128:131]"
    lines = [f"v_mov_b32 v{128 + i}, 0" for i in range(4)]
    # mc = 0 while m = -inf: the -m blocks start at -BIAS / scale_log2 and every row is flagged
    lines += [f"v_mov_b32 v{CB + i}, %[nbias]" for i in range(32)]
    lines += [f"v_mov_b32 v{M}, {NEG_INF}", f"v_mov_b32 v{M + 1}, {NEG_INF}"]
    lines += [f"v_mfma_f32_32x32x16_bf16 a[{16 * i}:{16 * i + 15}], {zero}, {zero}, 0" for i in range(8)]
    b = p_base(1)
    lines += [f"v_mfma_f32_32x32x16_bf16 v[{b + 16 * i}:{b + 16 * i + 15}], {zero}, {zero}, 0" for i in range(2)]
    lines += [f"v_mfma_f32_16x16x32_bf16 v[{TS + 4 * qb}:{TS + 4 * qb + 3}], {zero}, {zero}, 0" for qb in range(2)]
    lines.append("s_mov_b64 %[ninf], -1")
    return lines


def pv_only_block(ph):
    """The last PV, as the PV of an iteration of phase ph would run it."""
    pp = 1 - ph % 2
    sums = [rowsum_mfma(pp, qb, ks) for ks in range(4) for qb in range(2)]
    return stream(v_reads(), pp, ph, sums) + ["s_nop 11"]


def check_hazards(lines):
    """An MFMA result is not read by a VALU op within 12 instructions; a register an MFMA reads
    is not overwritten by an LDS read within 12 instructions; an exponential's result is not
    read by the next instruction; a dot2 result is read by another op only after 3 wait
    states; an LDS DMA load does not directly follow the write of m0."""
    last_write = {}
    last_exp = {}
    last_mfma_read = {}
    last_dot = {}
    last_valu = {}
    pending = []                                 # destination registers of LDS ops in flight
    last_m0 = -100
    for idx, l in enumerate(lines):
        op = l.split()[0] if l.split() else ""
        if op.startswith("s_") and op != "s_nop" and len(l.split()) > 1 and l.split()[1].rstrip(",") == "m0":
            last_m0 = idx
        if op.startswith("global_load_lds"):
            assert idx - last_m0 >= 2, (l, "m0 written by the previous instruction")
        if op == "s_waitcnt" and "lgkmcnt(" in l:
            n = int(l.split("lgkmcnt(")[1].split(")")[0])
            pending = pending[max(len(pending) - n, 0):]
        if op.startswith(("v_", "ds_")) and pending:
            srcs = l.replace(",", " ").split()[2:] if not op.startswith("ds_") else l.replace(",", " ").split()[1:]
            if op.startswith("ds_read") or op == "ds_bpermute_b32":
                srcs = l.replace(",", " ").split()[2:]
            for tok in srcs:
                tok = tok.lstrip("-")
                regs = set()
                if tok.startswith("v[") and ":" in tok:
                    lo_, hi_ = (int(x) for x in tok[2:].rstrip("]").split(":"))
                    regs = {f"v{x}" for x in range(lo_, hi_ + 1)}
                elif tok.startswith("v") and tok[1:].isdigit():
                    regs = {tok}
                for d in pending:
                    assert not (regs & d), (l, "reads an LDS result before its lgkmcnt wait")
        if op.startswith("ds_"):
            d = set()
            if op.startswith("ds_read") or op == "ds_bpermute_b32":
                dst = l.split()[1].rstrip(",")
                if dst.startswith("v["):
                    lo_, hi_ = (int(x) for x in dst[2:-1].split(":"))
                    d = {f"v{x}" for x in range(lo_, hi_ + 1)}
                else:
                    d = {dst}
            pending.append(d)
        if op.startswith("v_mfma"):
            for opnd in l.replace(",", " ").split()[2:5]:
                if opnd.startswith("v["):
                    lo_, hi_ = (int(x) for x in opnd[2:-1].split(":"))
                    for v in range(lo_, hi_ + 1):
                        if f"v{v}" in last_valu:
                            assert idx - last_valu[f"v{v}"] >= 4, (l, idx - last_valu[f"v{v}"], "MFMA reads a fresh VALU result")
            dst = l.split()[1].rstrip(",")
            lo = int(dst[2:].split(":")[0])
            for v in range(lo, lo + 16):
                last_write[dst[0] + str(v)] = idx
            a = l.split()[2].rstrip(",")
            if a.startswith("v["):
                alo = int(a[2:].split(":")[0])
                for v in range(alo, alo + 4):
                    last_mfma_read["v" + str(v)] = idx
            continue
        if op == "ds_read_b128":
            d = l.split()[1].rstrip(",")
            dlo = int(d[2:].split(":")[0])
            for v in range(dlo, dlo + 4):
                if "v" + str(v) in last_mfma_read:
                    assert idx - last_mfma_read["v" + str(v)] >= 12, (l, idx - last_mfma_read["v" + str(v)])
        if op.startswith("v_") and not op.startswith("v_mfma") and len(l.split()) > 1:
            dst = l.split()[1].rstrip(",")
            for v in ([dst] if not dst.startswith("v[") else [f"v{x}" for x in range(int(dst[2:].split(":")[0]), int(dst[:-1].split(":")[1]) + 1)]):
                if v in last_mfma_read:
                    assert idx - last_mfma_read[v] >= 12, (l, idx - last_mfma_read[v], "VALU overwrites an MFMA operand")
        if op.startswith("v_") or op.startswith("ds_"):
            toks = l.replace(",", " ").split()[2:] if not op.startswith("ds_") else l.replace(",", " ").split()[1:]
            for tok in toks:
                tok = tok.lstrip("-")
                if tok in last_write:
                    assert idx - last_write[tok] >= 12, (l, idx - last_write[tok])
                if tok in last_exp:
                    assert idx - last_exp[tok] >= 2, (l, idx - last_exp[tok])
            if op == "v_exp_f32":
                last_exp[l.split()[1].rstrip(",")] = idx
            if op.startswith("v_") and not op.startswith(("v_cmp", "v_readlane", "v_readfirstlane", "v_accvgpr_write")):
                last_valu[l.split()[1].rstrip(",")] = idx
            if op == "v_dot2_f32_bf16":
                last_dot[l.split()[1].rstrip(",")] = idx
            else:
                for tok in toks:
                    tok = tok.lstrip("-")
                    if tok in last_dot:
                        assert idx - last_dot[tok] >= 4, (l, idx - last_dot[tok])
        if op == "s_nop":
            n = int(l.split()[1]) + 1
            last_write = {k: v - n for k, v in last_write.items()}
            last_exp = {k: v - n for k, v in last_exp.items()}
            last_mfma_read = {k: v - n for k, v in last_mfma_read.items()}
            last_dot = {k: v - n for k, v in last_dot.items()}
            last_valu = {k: v - n for k, v in last_valu.items()}
            last_m0 -= n


KOFF, VOFF, SLOTL = 236, 240, 244                # lane offsets of the K and V^T tile loads, frame slots
CB = 202                                         # -(m + BIAS) / scale_log2 blocks, v[202:217] (qb 0) and v[218:233]
MT = 245                                         # mask word read from its AGPR
MKA, LANEA = 192, 224                            # mask words a[192 + 16 qb + j]; 8g, tq, bperm at a[224:227]
SEL = 228                                        # row-sum selector a[228:231] (A operand)
ACC = 246                                        # OR of the tile's P words (lazy test)
BIAS = 8                                         # P = 2^(s * scale_log2 - m - BIAS)


def set_mode(f8, scaled=False):
    """Program for the e4m3 cache (staged loads widened to bf16) or the bf16 cache; scaled: the
    bf16 cache holds its keys times scale_log2 (no product per score)."""
    global F8, SCALED
    F8 = f8
    SCALED = scaled


KTILE = 16384                                    # bytes of a K (or V^T) tile in LDS
NSLOT = 4                                        # ring slots of K and of V^T tiles


BASE = ((84, 86), (88, 90))                      # by parity: SGPR pairs of the K and V^T load bases
F8 = False                                       # program for the e4m3 cache (set by set_mode)
SCALED = False                                   # keys cached times scale_log2 (set by set_mode)
STAGE = 16384                                    # e4m3 staging slot: K tile (8 KB), then V^T tile (8 KB)
SK, SV = 234, 235                                # e4m3: this lane's staging read addresses (K, V^T)
WKA, WVA = 232, 236                              # e4m3: widened-chunk write addresses (AGPRs; lo, hi per load)


def tile_loads(ph):
    """Read index -> (m0 setup, load) of this wave's tile loads in iteration phase ph: bf16,
    four 1 KB K loads (after reads 1, 5, 9, 13) into ring slot ph + 2 and four V^T loads (after
    reads 17, 21, 25, 29) into slot ph + 1; e4m3, two of each (after reads 1, 3 and 5, 7:
    early, so that they land before the next iteration widens them) into staging slot ph mod 2.  m0 holds the LDS destination, the SGPR pair of parity ph mod 2
    the global tile base and v[236:243] the lane offsets."""
    par = ph % 2
    d = {}
    if F8:
        kinds = ((1, "ms", (ph % 2) * STAGE, BASE[par][0], KOFF), (5, "ms", (ph % 2) * STAGE + STAGE // 2, BASE[par][1], VOFF))
        n, step = 2, 2
    else:
        kinds = ((1, "mk", ((ph + 2) % NSLOT) * KTILE, BASE[par][0], KOFF),
                 (17, "mv", ((ph + 1) % NSLOT) * KTILE, BASE[par][1], VOFF))
        n, step = 4, 4
    for first, mbase, off, base, v0 in kinds:
        for i in range(n):
            setup = f"s_add_u32 m0, %[{mbase}], {off}" if i == 0 else "s_add_u32 m0, m0, 1024"
            d[first + step * i] = (setup, f"global_load_lds_dwordx4 v{v0 + i}, s[{base}:{base + 1}]")
    return d


def widen_block(ph):
    """e4m3, before the loop (ph = 0): this wave's staged bytes of K(0) and of the zeroed V^T(-1)
    (staging slot 0, the prologue's first loads) widened to bf16 into ring slots 0 and 3.  A
    staged 16-byte chunk c = 2p + h of a row holds, in the cache's byte order, elements
    32p + 8h + [0, 8) and 32p + 16 + 8h + [0, 8): the bf16 chunks 4p + h (lo) and 4p + 2 + h
    (hi), whose LDS addresses wait in a[232:239]."""
    stage = (ph % 2) * STAGE
    parts = [("K", i) for i in range(2)] + [("V", i) for i in range(2)]
    lines = []
    for j, (kind, i) in enumerate(parts):
        addr, off = (SK, stage + i * 1024) if kind == "K" else (SV, stage + i * 1024)
        lines.append(f"ds_read_b128 v[{128 + 4 * j}:{131 + 4 * j}], v{addr} offset:{off}")
    # the write addresses wait in AGPRs: copy this block's into the free temporaries
    waddr = {}
    for kind, i in parts:
        for half in range(2):
            src = (WKA if kind == "K" else WVA) + 2 * i + half
            waddr[(kind, i, half)] = f"v{TMP + len(waddr)}"
            lines.append(f"v_accvgpr_read_b32 {waddr[(kind, i, half)]}, a{src}")
    lines.append("s_waitcnt lgkmcnt(0)")
    for j in range(len(parts)):
        for dw in range(4):
            for sel in range(2):
                o = f"v{144 + 8 * j + 2 * dw + sel}"
                lines.append(f"v_cvt_scalef32_pk_bf16_fp8 {o}, v{128 + 4 * j + dw}, 1.0" + (" op_sel:[1,0,0]" if sel else ""))
    for j, (kind, i) in enumerate(parts):
        slot = ph % NSLOT if kind == "K" else (ph - 1) % NSLOT
        for half in range(2):
            lines.append(f"ds_write_b128 {waddr[(kind, i, half)]}, v[{144 + 8 * j + 4 * half}:{147 + 8 * j + 4 * half}] "
                         f"offset:{slot * KTILE}")
    lines.append("s_waitcnt lgkmcnt(0)")
    return lines


def widen_units(ph, pc):
    """e4m3, iteration phase ph: this wave's staged bytes of K(t+1) and V^T(t) (staging slot
    (ph + 1) mod 2, loaded by the previous iteration) widened to bf16 into ring slots ph + 1 (K)
    and ph (V^T), in the gaps before the softmax: as (first gap, unit) pairs for stream().
    Registers: P buffer pc, whose P(t-2) is dead until the softmax writes P(t) there, holds
    chunk j = (K0, K1, V0, V1) in its 8 registers R..R+7: the staged 16 bytes are read into
    R+4..R+7 and widened in place (bf16 pair 2dw + sel from staged word dw: each word is read
    by both of its conversions before a later one overwrites it); the temporaries hold the
    write addresses.  K is widened first: its loads were issued earliest.  The eight widened
    writes go one per MFMA pair, pairs 2 to 9, each after the pair's fragment reads: LDS ops
    complete in order, and writes issued ahead of fragment reads (two per gap, as first
    written) held those reads back; placed behind them the 14B call ran 3-4 % faster."""
    stage = ((ph + 1) % 2) * STAGE
    base = p_base(pc)
    units = []

    def at(gap, *ins):
        units.append((gap, list(ins)))

    def addresses(kind, gap):                  # write addresses of (kind, 0) and (kind, 1)
        a0, t0 = (WKA, TMP) if kind == "K" else (WVA, TMP + 4)
        for h in range(2):
            at(gap, *[f"v_accvgpr_read_b32 v{t0 + 2 * h + x}, a{a0 + 2 * h + x}" for x in range(2)])

    def read(j, gap):
        kind, i = ("K", "K", "V", "V")[j], j % 2
        R = base + 8 * j
        at(gap, f"s_waitcnt vmcnt(@P{j})",
           (f"ds_read_b128 v[{R + 4}:{R + 7}], v{SK if kind == 'K' else SV} offset:{stage + i * 1024}", f"W{j}"))

    def widen(j, gap):
        kind = ("K", "K", "V", "V")[j]
        R = base + 8 * j
        slot = (ph + 1) % NSLOT if kind == "K" else ph % NSLOT
        cv = [f"v_cvt_scalef32_pk_bf16_fp8 v{R + 2 * dw + sel}, v{R + 4 + dw}, 1.0" + (" op_sel:[1,0,0]" if sel else "")
              for dw in range(4) for sel in range(2)]
        at(gap, (f"s_waitcnt lgkmcnt(@W{j})", None), cv[0], cv[1])
        for k in range(2, 8, 2):
            at(gap, cv[k], cv[k + 1])
        for h in range(2):
            at(5 + 4 * j + 2 * h, LATE,
               f"ds_write_b128 v{TMP + 2 * j + h}, v[{R + 4 * h}:{R + 4 * h + 3}] offset:{slot * KTILE}")

    # the four reads first (the loads landed most of an iteration ago), each chunk's conversion
    # a few gaps after its read (LDS latency), its two writes in later pairs
    addresses("K", 0)
    for j in range(4):
        read(j, 1 + j)
    addresses("V", 2)
    for j in range(4):
        widen(j, 2 + 2 * j)
    return units


def k_setup(par, ahead):
    """Global base of the loads of K (t + ahead) for the iteration of parity par, as
    load_setup does it, and besides it ov, the V^T offset of the same tile (its V^T base one
    iteration later: V^T runs one tile behind K).  Units."""
    units = load_setup("K", par, ahead)
    i = units.index(NEXT_GAP)
    return units[:i + 1] + [[f"s_lshl_b32 %[y], %[kk], {6 if F8 else 7}"],
                            ["s_mul_i32 %[x], %[x], %[slotb]"],
                            ["s_add_u32 %[ov], %[x], %[y]"],
                            [f"s_lshl_b32 %[y], %[kk], {13 if F8 else 14}"],
                            ["s_add_u32 %[x], %[x], %[y]"],
                            units[-1]]


def v_setup(par):
    """Global base of the V^T loads of the next iteration of parity par: V^T (t + 2) is the K
    tile of the previous iteration's k_setup, whose V^T offset is ov."""
    b = BASE[par][1]
    return [[f"s_add_u32 s{b}, %[vblo], %[ov]", f"s_addc_u32 s{b + 1}, %[vbhi], 0"]]


def cursor_shift():
    """The walk cursor of tile t+1 is the K cursor of two iterations before (held in vk, vf
    for one iteration): sk, sf <- vk, vf <- kk, kf, before k_setup advances kk, kf."""
    return [["s_mov_b32 %[sk], %[vk]"], ["s_mov_b32 %[sf], %[vf]"],
            ["s_mov_b32 %[vk], %[kk]"], ["s_mov_b32 %[vf], %[kf]"]]


def load_setup(kind, par, ahead):
    """Global base of the loads of K (t + ahead) or V^T (t + ahead) for the iteration of parity
    par: the cursor advances when that tile exists (otherwise the loads repeat the last tile,
    a valid address, into the free slot, so every iteration issues eight loads and one vmcnt
    serves all).  Returned as units (instruction lists closed in their use of SCC)."""
    f, k, colb, blo, bhi, base = (
        ("kf", "kk", 13 if F8 else 14, "kblo", "kbhi", BASE[par][0]) if kind == "K"
        else ("vf", "vk", 6 if F8 else 7, "vblo", "vbhi", BASE[par][1]))
    return [[f"s_add_u32 %[x], %[t], {ahead}", "s_cmp_lt_u32 %[x], %[n]", "s_cselect_b32 %[y], 1, 0"],
            [f"s_add_u32 %[{k}], %[{k}], %[y]"],
            [f"s_cmp_eq_u32 %[{k}], %[tpf]", f"s_cselect_b32 %[{k}], 0, %[{k}]", f"s_addc_u32 %[{f}], %[{f}], 0"],
            [f"v_readlane_b32 %[x], v{SLOTL}, %[{f}]"], NEXT_GAP,     # its SGPR result is read
            # about 20 cycles later at the earliest: the wait overlaps the next MFMA
            # tile offset in the (layer, head) block: slot * slot bytes + tile (64 K rows or 64 V^T
            # columns of 2 bytes, or 1 byte in e4m3)
            [f"s_lshl_b32 %[y], %[{k}], {colb}"],
            ["s_mul_i32 %[x], %[x], %[slotb]"],
            ["s_add_u32 %[x], %[x], %[y]"],
            [f"s_add_u32 s{base}, %[{blo}], %[x]", f"s_addc_u32 s{base + 1}, %[{bhi}], 0"]]


def walk_setup(par, advance):
    """Tile t+1 of the softmax walk (tile 0 when advance is False): cursor, valid keys, own frame
    index tk, and mflag of parity par (1: ragged or partly causal, take the masked block).
    Returned as units."""
    units = []
    if advance:
        units += [["s_add_u32 %[x], %[t], 1", "s_cmp_lt_u32 %[x], %[n]", "s_cselect_b32 %[y], 1, 0"],
                  ["s_add_u32 %[sk], %[sk], %[y]"],
                  ["s_cmp_eq_u32 %[sk], %[tpf]", "s_cselect_b32 %[sk], 0, %[sk]", "s_addc_u32 %[sf], %[sf], 0"]]
    units += [["s_lshl_b32 %[x], %[sk], 6"], ["s_sub_i32 %[nvalid], %[N], %[x]"],
              ["s_min_i32 %[nvalid], %[nvalid], 64"],
              ["s_sub_i32 %[tk], %[sf], %[nshared]"],
              ["s_cmp_lt_i32 %[nvalid], 64", f"s_cselect_b32 %[mflag{par}], 1, 0"],
              ["s_cmp_gt_i32 %[tk], %[tqw]", "s_cselect_b32 %[x], 1, 0"],
              [f"s_or_b32 %[mflag{par}], %[mflag{par}], %[x]"]]
    return units


def iteration(ph):
    """Iteration t < n of phase ph = t mod NSLOT (P buffer pp = 1 - ph mod 2 read by PV(t-1),
    P(t) written into the other).  The masked tile block and the rescale are out of line."""
    par, tag = ph % 2, "abcd"[ph]
    # bf16: the loads of iteration t-2 (K(t), V^T(t-1)) are in; e4m3: this wave's widening of
    # them (the previous iteration's stream) is written.  Every wave is done with iteration t-1.
    return ([] if F8 else ["s_waitcnt vmcnt(8)"]) + ["s_barrier",
            f"s_cmp_eq_u32 %[mflag{par}], 0", f"s_cbranch_scc0 .Lw64_m{tag}_%="] + \
        tile_block(ph, False) + \
        [f".Lw64_td{tag}_%=:",
         "s_cmp_eq_u64 %[trig], 0", f"s_cbranch_scc0 .Lw64_r{tag}_%=",
         f".Lw64_nr{tag}_%=:",
         "s_add_u32 %[t], %[t], 1"]


def out_of_line(ph):
    par, tag = ph % 2, "abcd"[ph]
    pc = par                                     # P buffer written by iteration phase ph
    return ([f".Lw64_m{tag}_%=:"] + tile_block(ph, True) + [f"s_branch .Lw64_td{tag}_%=",
            f".Lw64_r{tag}_%=:", f"s_cmp_eq_u32 %[mflag{par}], 0", f"s_cbranch_scc1 .Lw64_ru{tag}_%="]
            + rare_block(pc, True) + [f"s_branch .Lw64_nr{tag}_%=", f".Lw64_ru{tag}_%=:"]
            + rare_block(pc, False) + [f"s_branch .Lw64_nr{tag}_%="])


def loop_program():
    """The whole tile loop: iterations t = 0 .. n-1 (NSLOT per pass, so that ring slots, P
    buffer and set-up parity are fixed in each copy), then the last PV.  m0 is saved and
    restored."""
    set_mode(F8, SCALED)
    RARE_ID[0] = 0
    lines = ["s_mov_b32 %[m0save], m0"] + init_block()
    # V^T base of tile 1 from the K cursor (tile 1), then vk, vf <- kk, kf and K advances to tile 2
    b = BASE[0][1]
    v1 = [f"v_readlane_b32 %[x], v{SLOTL}, %[kf]", "s_mul_i32 %[x], %[x], %[slotb]",
          f"s_lshl_b32 %[y], %[kk], {6 if F8 else 7}", "s_add_u32 %[x], %[x], %[y]",
          f"s_add_u32 s{b}, %[vblo], %[x]", f"s_addc_u32 s{b + 1}, %[vbhi], 0"]
    lines += sum((u for u in walk_setup(0, False) if u != NEXT_GAP), []) + v1 + \
        ["s_mov_b32 %[vk], %[kk]", "s_mov_b32 %[vf], %[kf]"] + \
        sum((u for u in k_setup(0, 2) if u != NEXT_GAP), [])
    if F8:
        # staging slot 0 (K(0) and a zeroed V^T half, the prologue's first loads) into ring slots
        # 0 and 3; slot 1 (K(1), V^T(0)) is widened by iteration 0
        lines += ["s_waitcnt vmcnt(4)"] + widen_block(0)
    lines += [".Lw64_loop_%=:"]
    for ph in range(NSLOT):
        lines += iteration(ph)
        if ph < NSLOT - 1:
            lines += ["s_cmp_lt_u32 %[t], %[n]", "s_cbranch_scc0 .Lw64_end_%="]
    lines += ["s_cmp_lt_u32 %[t], %[n]", "s_cbranch_scc1 .Lw64_loop_%=",
              ".Lw64_end_%=:", "s_waitcnt vmcnt(0)", f"s_and_b32 %[x], %[n], {NSLOT - 1}"]
    for ph in range(1, NSLOT):
        lines += [f"s_cmp_eq_u32 %[x], {ph}", f"s_cbranch_scc1 .Lw64_pv{ph}_%="]
    for ph in range(NSLOT):
        lines += ([f".Lw64_pv{ph}_%=:"] if ph else []) + ["s_barrier"] + pv_only_block(ph) + \
            ["s_branch .Lw64_fin_%="]
    for ph in range(NSLOT):
        lines += out_of_line(ph)
    lines += [".Lw64_fin_%=:", "s_mov_b32 m0, %[m0save]"]
    return lines


def basic_blocks(lines):
    """Split a program into basic blocks: (label or None, instructions, successor labels).  A
    block ends at a label or after a branch; s_branch has only its target as successor, a
    conditional branch its target and the next block, any other end the next block."""
    blocks, cur, lab = [], [], None
    for l in lines + [".Lprogram_end:"]:
        if l.startswith(".L"):
            if cur or lab is not None:
                blocks.append([lab, cur])
            lab, cur = l.rstrip(":"), []
            continue
        cur.append(l)
        if l.split()[0].startswith(("s_branch", "s_cbranch")):
            blocks.append([lab, cur])
            lab, cur = None, []
    out = []
    for i, (lab, ins) in enumerate(blocks):
        succ = []
        last = ins[-1].split() if ins else [""]
        nxt = blocks[i + 1][0] if i + 1 < len(blocks) else None
        if last[0].startswith(("s_branch", "s_cbranch")):
            succ.append(last[-1])
        if not last[0].startswith("s_branch") and i + 1 < len(blocks):
            if nxt is None:                      # an unlabelled block after a conditional branch
                nxt = blocks[i + 1][0] = f".Lfall{i + 1}"
            succ.append(nxt)
        out.append((lab if lab is not None else f".Lentry{i}", ins, succ))
    # an unlabelled block reached by fall-through got its name above
    return [(blocks[i][0] or lab, ins, succ) for i, (lab, ins, succ) in enumerate(out)]


def check_paths(lines, history=64, depth=3):
    """check_hazards along the control flow: for every chain of up to `depth` basic blocks
    linked by a branch or a fall-through, the last `history` instructions of the chain's first
    blocks followed by the whole last block."""
    blocks = basic_blocks(lines)
    by_label = {lab: (ins, succ) for lab, ins, succ in blocks}
    preds = {lab: [] for lab, _, _ in blocks}
    for lab, _, succ in blocks:
        for t in succ:
            if t in preds:
                preds[t].append(lab)
    checked = set()

    def walk(lab, tail, d):
        key = (lab, d, tuple(tail[-history:]))
        if key in checked:
            return
        checked.add(key)
        check_hazards(tail[-history:] + by_label[lab][0])
        if d < depth:
            for s in by_label[lab][1]:
                if s in by_label:
                    walk(s, (tail + by_label[lab][0])[-history:], d + 1)

    for lab, ins, _ in blocks:
        walk(lab, [], 1)


def check_staging(iterations=10, masked=(2, 5)):
    """e4m3: run the loads, waits and LDS traffic of the tile loop as one wave executes them
    (the prologue's six loads, the widening before the loop, iterations 0 .. iterations-1,
    masked at the given ones, the last PV) and check the data each LDS read finds: a staged
    chunk is read only once its load is counted complete by a vmcnt wait and holds the tile the
    widening expects (iteration t widens K(t+1) and V^T(t)); the fragment reads of iteration t
    find K(t) and V^T(t-1) in the bf16 ring, the last PV V^T(n-1), written by the widening
    before a barrier; a widened write goes into a ring slot only after a barrier has passed since
    the slot's last read.  The other waves' share is the same with its own addresses, and the
    barrier at each iteration's top orders the waves."""
    assert F8
    pending = [((0, 0), ("K", 0)), ((0, 1), ("K", 0)), ((1, 0), ("K", 1)), ((1, 1), ("K", 1)),
               ((1, 8), ("V", 0)), ((1, 9), ("V", 0))]
    staged = {(0, 8): ("V", -1), (0, 9): ("V", -1)}          # zeroed by the prologue: V^T(-1)
    ring, regs, addr_kind, last_read = {}, {}, {}, {}
    m0, barriers = None, 0

    def run(lines, t, expect_k, expect_v):
        nonlocal pending, m0, barriers
        for l in lines:
            tok = l.replace(",", " ").split()
            if not tok or l.startswith(".L"):
                continue
            op = tok[0]
            if op == "s_barrier":
                barriers += 1
            elif op == "s_add_u32" and tok[1] == "m0":
                m0 = int(tok[3]) if tok[2] == "%[ms]" else (m0 + int(tok[3]) if tok[2] == "m0" else None)
            elif op.startswith("global_load_lds"):
                part = (m0 // STAGE, (m0 % STAGE) // 1024)
                what = ("K", t + 2) if tok[1] in (f"v{KOFF}", f"v{KOFF + 1}") else ("V", t + 1)
                pending.append((part, what))
                staged.pop(part, None)
            elif op == "s_waitcnt" and "vmcnt(" in l:
                n = int(l.split("vmcnt(")[1].split(")")[0])
                for part, what in (pending[:len(pending) - n] if n else pending):
                    staged[part] = what
                pending = pending[len(pending) - n:] if n else []
            elif op == "v_accvgpr_read_b32" and tok[2] in [f"a{WKA + i}" for i in range(4)] + [f"a{WVA + i}" for i in range(4)]:
                addr_kind[tok[1]] = "K" if int(tok[2][1:]) < WVA else "V"
            elif op == "ds_read_b128":
                lo = int(tok[1][2:].split(":")[0])
                off = int(tok[3].split(":")[1])
                if tok[2] in (f"v{SK}", f"v{SV}"):
                    part = (off // STAGE, (off % STAGE) // 1024 + (8 if tok[2] == f"v{SV}" else 0))
                    assert part in staged, (t, l, "reads a staged chunk whose load may not have landed")
                    want = expect_k if tok[2] == f"v{SK}" else expect_v
                    assert staged[part] == want, (t, l, staged[part], want)
                    for r in range(lo, lo + 4):
                        regs[r] = staged[part]
                else:
                    kind = "K" if KADDR <= int(tok[2][1:]) < KADDR + 8 else "V"
                    want = ("K", t) if kind == "K" else ("V", t - 1)
                    what, when = ring.get((kind, off // KTILE), (None, None))
                    assert what == want, (t, l, what, want)
                    assert when < barriers, (t, l, "reads a widened tile no barrier has passed since")
                    last_read[(kind, off // KTILE)] = barriers
            elif op == "v_cvt_scalef32_pk_bf16_fp8":
                regs[int(tok[1][1:])] = regs[int(tok[2][1:])]
            elif op == "ds_write_b128":
                lo = int(tok[2][2:].split(":")[0])
                vals = {regs.get(r) for r in range(lo, lo + 4)}
                assert len(vals) == 1, (t, l, vals)
                what = vals.pop()
                assert what is not None, (t, l, "writes registers no widening has filled")
                assert what[0] == addr_kind[tok[1]], (t, l, what)
                key = (what[0], int(tok[3].split(":")[1]) // KTILE)
                assert last_read.get(key, -1) < barriers, (t, l, "widens into a slot read since the last barrier")
                ring[key] = (what, barriers)

    lines = loop_program()
    pre = lines[:lines.index(".Lw64_loop_%=:")]
    run(pre, -1, ("K", 0), ("V", -1))
    for t in range(iterations):
        ph = t % NSLOT
        body = tile_block(ph, t in masked)
        run(["s_barrier"] + body, t, ("K", t + 1), ("V", t))
    ph = iterations % NSLOT
    run(["s_waitcnt vmcnt(0)", "s_barrier"] + pv_only_block(ph), iterations, None, None)


def check_ring(iterations=10, masked=(2, 5), rare=(3, 5)):
    """bf16: run the tile loads, waits, barriers and LDS reads of the tile loop as one wave
    executes them (the prologue's loads of K(0) and K(1) into ring slots 0 and 1 and of V^T(0)
    into slot 0 with V^T(-1) zeroed in slot 3, iterations 0 .. iterations-1, masked and rescaled
    at the given ones, the last PV) and check the ring protocol.  A fragment read of iteration t
    finds K(t) (V^T(t-1)) in its slot: this wave's four 1 KB pieces of that tile were loaded
    there, counted complete by a vmcnt wait, and a barrier has passed since (every wave runs
    this program on its own pieces, so then every piece is in).  A tile load goes into a slot
    only after a barrier has passed since the slot's last read, and no LDS op is in flight at a
    barrier."""
    assert not F8
    pending = [((kind, slot, p), what) for kind, slot, what in
               (("K", 0, ("K", 0)), ("K", 1, ("K", 1)), ("V", 0, ("V", 0))) for p in range(4)]
    done, visible, last_read = {}, {("V", 3): ("V", -1)}, {}
    state = {"barriers": 0, "lds": 0, "m0": None}

    def run(lines, t):
        nonlocal pending
        for l in lines:
            tok = l.replace(",", " ").split()
            if not tok or l.startswith(".L"):
                continue
            op = tok[0]
            if op == "s_add_u32" and tok[1] == "m0":
                if tok[2] in ("%[mk]", "%[mv]"):
                    state["m0"] = ("K" if tok[2] == "%[mk]" else "V", int(tok[3]))
                elif tok[2] == "m0" and state["m0"]:
                    state["m0"] = (state["m0"][0], state["m0"][1] + int(tok[3]))
                else:
                    state["m0"] = None
            elif op.startswith("global_load_lds"):
                assert state["m0"], (t, l, "m0 does not hold a ring address")
                kind, off = state["m0"]
                key = (kind, off // KTILE)
                assert last_read.get(key, -1) < state["barriers"], (t, l, "a load into a slot read since the last barrier")
                pending.append(((kind, off // KTILE, (off % KTILE) // 1024), ("K", t + 2) if kind == "K" else ("V", t + 1)))
                visible.pop(key, None)
            elif op == "s_waitcnt" and "vmcnt(" in l:
                n = int(l.split("vmcnt(")[1].split(")")[0])
                for piece, what in pending[:max(0, len(pending) - n)]:
                    done[piece] = what
                pending = pending[max(0, len(pending) - n):]
            elif op == "s_waitcnt" and "lgkmcnt(" in l:
                state["lds"] = min(state["lds"], int(l.split("lgkmcnt(")[1].split(")")[0]))
            elif op == "s_barrier":
                assert state["lds"] == 0, (t, "LDS ops in flight at a barrier")
                state["barriers"] += 1
                busy = {piece[:2] for piece, _ in pending}
                for kind in "KV":
                    for sl in range(NSLOT):
                        w = {done.get((kind, sl, p)) for p in range(4)}
                        if len(w) == 1 and None not in w and (kind, sl) not in busy:
                            visible[(kind, sl)] = w.pop()
            elif op == "ds_read_b128":
                a, off = int(tok[2][1:]), int(tok[3].split(":")[1])
                kind = "K" if KADDR <= a < KADDR + 8 else "V"
                assert kind == "K" or VADDR <= a < VADDR + 4, (t, l)
                key = (kind, off // KTILE)
                want = ("K", t) if kind == "K" else ("V", t - 1)
                assert visible.get(key) == want, (t, l, visible.get(key), want)
                last_read[key] = state["barriers"]
                state["lds"] += 1
            elif op.startswith("ds_"):
                state["lds"] += 1

    lines = loop_program()
    run(lines[:lines.index(".Lw64_loop_%=:")], -1)
    for t in range(iterations):
        ph = t % NSLOT
        top = iteration(ph)
        top = top[:next(i for i, l in enumerate(top) if l.startswith("s_cbranch_scc0 .Lw64_m")) + 1]
        body = tile_block(ph, t in masked) + (rare_block(ph % 2, t in masked) if t in rare else [])
        run(top + body, t)
    run(["s_waitcnt vmcnt(0)", "s_barrier"] + pv_only_block(iterations % NSLOT), iterations)


def emit(name, lines):
    check_hazards([l for l in lines if not l.startswith(".L")])
    check_paths(lines)
    body = " \\\n".join(f'  "{l}\\n\\t"' for l in lines)
    return f"#define {name} \\\n{body}\n"


def main():
    out = ["// Generated by gen_attn_w64.py; do not edit.  The tile loop of the 64-row attention",
           "// kernel as one asm program (register plan, blocks and hazard rules in the generator).", ""]
    set_mode(False)
    check_ring()
    out.append(emit("SDV2_W64_LOOP", loop_program()))
    set_mode(False, scaled=True)
    check_ring()
    out.append(emit("SDV2_W64_LOOP_SK", loop_program()))
    set_mode(True, scaled=True)
    check_staging()
    out.append(emit("SDV2_W64_LOOP_FP8", loop_program()))
    set_mode(False)
    sys.stdout.write("\n".join(out))


if __name__ == "__main__":
    main()
