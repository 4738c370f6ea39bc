"""Writes attn_w64_asm.h: the per-tile instruction streams of the 64-row attention kernel.

Run from this directory (`python3 gen_attn_w64.py > attn_w64_asm.h`); the header is committed
and a host test checks that it matches this script's output.

One wave owns 64 query rows (two 32-row blocks qb) of one (element, head).  Per 64-key tile it
issues 64 MFMAs 32x32x16 bf16 fed by 32 LDS fragment reads (each read feeds both row blocks):
  QK:  S^T[kb][qb] = K[kb] Q^T[qb]      16 K reads (kb-major, 8 k steps each)
  PV:  O^T[db][qb] += V^T[db] P^T[qb]   16 V^T reads (key step ks-major, d block db)
and, interleaved with the PV MFMAs, the softmax of the tile's S: exp2(S*scale_log2 - m) rounded
to bf16 P^T words for the next tile's PV, with per-lane tile sums by dot2 over the packed P.

Blocks (one asm statement each; every state register is an asm operand, so the compiler never
moves them):
  TILE_P{pp}, TILE_MASKED_P{pp}  QK(t), PV(t-1) with P buffer pp, softmax(t) into buffer 1-pp,
                                 the lazy test (trig != 0: some lane's tile sum left [0, 256]),
                                 l += tile sums when trig == 0, LDS address steps
  RARE_P{pc}, RARE_MASKED_P{pc}  the rescale: masked row max, m, alpha, O and l scaled, P of
                                 the tile recomputed into buffer pc, l += its sums
  PV_ONLY_P{pp}                  the last PV
The masked variants AND every P word with a ragged-tile mask (keys >= nvalid) and a per-row-
block causal mask (own frame tk after the row's frame), both computed at the block start.

Register plan (per lane):
  a[0:127]    O^T  o[db][qb] at a[(2db+qb)*16 .. +15]
  a[128:191]  Q^T  q[qb][kd] at a[128 + (8qb+kd)*4 .. +3]
  v[0:63]     S^T  s[kb][qb] at v[(2kb+qb)*16 .. +15]
  v[64:127]   P^T  two buffers, p[qb][ks] at base + (4qb+ks)*4, base 64 or 96
  v[128:175]  fragment ring, 12 slots of 4 (also DMA offsets and rare-path temporaries)
  v[176:183]  K fragment LDS addresses per k step kd;  v[184:187] V^T addresses per key step
  v[188:199]  temporaries
  v[200:201]  m per qb (running max, log2 units);  v[202:205] tile sums (two per qb)
  v[206:221]  ragged masks of the 16 P words of a row block;  v[222:223] causal mask per qb
  v[224] 8g;  v[225:226] frame of the lane's row per qb;  v[227] (lane ^ 32) * 4
  v[228:229]  l per qb;  v[230:237] K and V^T lane offsets of the tile loads;  v238 frame slots

Hazards kept by construction (gfx950, counted in issued instructions): an MFMA result is read
by no VALU or MFMA A/B operand within 12 instructions (checked below; S of kb = 1 is complete
after MFMA 31 and first read at MFMA 48; the rare block starts with 16 wait states); VALU-
written P words are read by MFMAs of the next tile only; an exponential's result is read at
least one instruction later; a dot2 result is read by an instruction other than the next
dot2 of the same sum only after 3 wait states (gfx950 does not interlock it: reading the sums
right after the last dot2 lost its update, measured);
a fragment slot is refilled at least 12 instructions after the
last MFMA that reads it (an MFMA may read its A operand after issue, so 8 reads in flight use
a ring of 12 slots);
same-accumulator MFMAs chain back to back (allowed); VOP3 forms read at most one SGPR.
"""
import sys

KA = 8                                           # fragment reads in flight
RING = 12                                        # fragment slots: a slot is refilled 4 reads after its last use
FR, KADDR, VADDR = 128, 176, 184
TMP, M, TS, RMASK, CMASK, G8, TQ, BPERM, L = 188, 200, 202, 206, 222, 224, 225, 227, 228
NEG_INF = "0xff800000"


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
    return [("K", kb, kd) for kb in range(2) for kd in range(8)]


def v_reads():
    return [("V", db, ks) for ks in range(4) for db in range(4)]


def read_instr(r, slot):
    if r[0] == "K":
        _, kb, kd = r
        return f"ds_read_b128 {frag(slot)}, v{KADDR + kd} offset:{kb * 8192}"
    _, db, ks = r
    return f"ds_read_b128 {frag(slot)}, v{VADDR + ks} offset:{db * 4096}"


def mfma_pair(r, slot, pp):
    out = []
    if r[0] == "K":
        _, kb, kd = r
        for qb in range(2):
            c = "0" if kd == 0 else s_reg(kb, qb)
            out.append(f"v_mfma_f32_32x32x16_bf16 {s_reg(kb, qb)}, {frag(slot)}, {q_reg(qb, kd)}, {c}")
    else:
        _, db, ks = r
        for qb in range(2):
            out.append(f"v_mfma_f32_32x32x16_bf16 {o_reg(db, qb)}, {frag(slot)}, {p_reg(pp, qb, ks)}, {o_reg(db, qb)}")
    return out


def softmax_ops(pc, masked, qbs=(0, 1), mreg=None, sums=None):
    """Groups of 4 values (kb-major, so the kb = 0 half only needs the first 16 QK MFMAs):
    4 FMAs, 4 exponentials, 2 packs into P words (masked: AND with the word's ragged mask and
    the row block's causal mask), 2 dot2 row sums into the two sums of the row block.  mreg(qb): register holding m; sums(qb, i):
    the two tile-sum accumulators."""
    mreg = mreg or (lambda qb: f"v{M + qb}")
    sums = sums or (lambda qb, i: f"v{TS + 2 * qb + i}")
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
                    for j in range(4):
                        ops.append(f"v_fma_f32 {t[j]}, {s_elem(kb, qb, vs[j])}, %[sl], -{mreg(qb)}")
                    for j in range(4):
                        ops.append(f"v_exp_f32 {t[j]}, {t[j]}")
                    words = [p_word(pc, qb, ks, w0), p_word(pc, qb, ks, w0 + 1)]
                    ops.append(f"v_cvt_pk_bf16_f32 {words[0]}, {t[0]}, {t[1]}")
                    ops.append(f"v_cvt_pk_bf16_f32 {words[1]}, {t[2]}, {t[3]}")
                    if masked:
                        for wi, w in enumerate(words):
                            j = ks * 4 + w0 + wi
                            ops.append(f"v_and_b32 {w}, {w}, v{RMASK + j}")
                            ops.append(f"v_and_b32 {w}, {w}, v{CMASK + qb}")
                    # word 0 into sum 0, word 1 into sum 1: a sum is accumulated again only
                    # one group (>= 10 instructions) later (dependent dot2 need spacing)
                    for i, wd in enumerate(words):
                        acc = sums(qb, i)
                        ops.append(f"v_dot2_f32_bf16 {acc}, {wd}, %[ones], {acc}")
    return ops


def mask_setup():
    """Ragged masks: low half of word j valid iff 8g + key(j) < nvalid, high half iff
    8g + key(j) + 1 < nvalid.  Causal mask of qb: all ones iff tk <= frame of the row."""
    lines = [f"v_mov_b32 v{TMP + 2}, 0xffff", f"v_mov_b32 v{TMP + 3}, 0xffff0000", f"v_mov_b32 v{TMP + 4}, -1"]
    for j in range(16):
        c = word_key(j)
        lines += [f"s_sub_i32 %[stmp], %[nvalid], {c}",
                  f"v_cmp_gt_i32 vcc, %[stmp], v{G8}",
                  f"v_cndmask_b32 v{TMP}, 0, v{TMP + 2}, vcc",
                  f"s_sub_i32 %[stmp], %[nvalid], {c + 1}",
                  f"v_cmp_gt_i32 vcc, %[stmp], v{G8}",
                  f"v_cndmask_b32 v{TMP + 1}, 0, v{TMP + 3}, vcc",
                  f"v_or_b32 v{RMASK + j}, v{TMP}, v{TMP + 1}"]
    for qb in range(2):
        lines += [f"v_cmp_le_i32 vcc, %[tk], v{TQ + qb}",
                  f"v_cndmask_b32 v{CMASK + qb}, 0, v{TMP + 4}, vcc"]
    return lines


def stream(reads, pp, valu):
    """Reads KA ahead of their MFMAs; VALU ops spread evenly over the PV MFMAs."""
    lines = []
    for i in range(min(KA, len(reads))):
        lines.append(read_instr(reads[i], i % RING))
    issued = min(KA, len(reads))
    pv_first = next(i for i, r in enumerate(reads) if r[0] == "V")
    n_pv_mfma = 2 * (len(reads) - pv_first)
    per = [0] * n_pv_mfma
    for i in range(len(valu)):
        per[i * n_pv_mfma // len(valu)] += 1
    vi = 0
    for i, r in enumerate(reads):
        lines.append(f"s_waitcnt lgkmcnt({min(issued - (i + 1), 15)})")
        for j, m in enumerate(mfma_pair(r, i % RING, pp)):
            lines.append(m)
            if i >= pv_first:
                k = 2 * (i - pv_first) + j
                for _ in range(per[k]):
                    lines.append(valu[vi])
                    vi += 1
        if i + KA < len(reads):
            lines.append(read_instr(reads[i + KA], (i + KA) % RING))
            issued += 1
    assert vi == len(valu)
    lines.append("s_waitcnt lgkmcnt(0)")
    return lines


def tile_block(pp, masked, tag=""):
    pc = 1 - pp
    lines = mask_setup() if masked else []
    lines += [f"v_mov_b32 v{TS + i}, 0" for i in range(4)]
    lines += stream(k_reads() + v_reads(), pp, softmax_ops(pc, masked))
    # lazy test and the common-path row sums (a dot2 result is read by another VALU op only
    # after 3 wait states)
    lines += ["s_nop 3",
              f"v_add_f32 v{TMP}, v{TS}, v{TS + 1}",
              f"v_add_f32 v{TMP + 1}, v{TS + 2}, v{TS + 3}",
              f"v_cmp_nge_f32 vcc, 0x43800000, v{TMP}",
              "s_mov_b64 %[trig], vcc",
              f"v_cmp_nge_f32 vcc, 0x43800000, v{TMP + 1}",
              "s_or_b64 %[trig], %[trig], vcc",
              "s_cmp_eq_u64 %[trig], 0",
              f"s_cbranch_scc0 .Lw64_keep{tag}_%=",
              f"v_add_f32 v{L}, v{L}, v{TMP}",
              f"v_add_f32 v{L + 1}, v{L + 1}, v{TMP + 1}",
              f".Lw64_keep{tag}_%=:"]
    lines += [f"v_add_u32 v{KADDR + kd}, %[kstep], v{KADDR + kd}" for kd in range(8)]
    lines += [f"v_add_u32 v{VADDR + ks}, %[vstep], v{VADDR + ks}" for ks in range(4)]
    lines.append("s_nop 11")
    return lines


def rare_block(pc, masked):
    mx, y, mn, al, mm, t0, t1, ninf = (f"v{x}" for x in range(128, 136))
    lines = ["s_nop 15", f"v_mov_b32 {ninf}, {NEG_INF}"]
    for qb in range(2):
        lines.append(f"v_mov_b32 {mx}, {NEG_INF}")
        for j in range(16):
            kb, v = j >> 3, ((j >> 2) & 1) * 8 + 2 * (j & 3)
            lo, hi = s_elem(kb, qb, v), s_elem(kb, qb, v + 1)
            if masked:
                lines += [f"v_and_b32 {t0}, v{RMASK + j}, v{CMASK + qb}",
                          f"v_and_b32 {t1}, 0xffff, {t0}",
                          f"v_cmp_ne_u32 vcc, 0, {t1}",
                          f"v_cndmask_b32 {t1}, {ninf}, {lo}, vcc",
                          f"v_max_f32 {mx}, {mx}, {t1}",
                          f"v_cmp_lt_u32 vcc, 0xffff, {t0}",
                          f"v_cndmask_b32 {t1}, {ninf}, {hi}, vcc",
                          f"v_max_f32 {mx}, {mx}, {t1}"]
            else:
                lines.append(f"v_max3_f32 {mx}, {mx}, {lo}, {hi}")
        lines += [f"ds_bpermute_b32 {y}, v{BPERM}, {mx}",
                  "s_waitcnt lgkmcnt(0)",
                  f"v_max_f32 {mx}, {mx}, {y}",
                  f"v_mul_f32 {t0}, %[sl], {mx}",
                  f"v_max_f32 {mn}, v{M + qb}, {t0}",                 # m_new
                  f"v_sub_f32 {t0}, v{M + qb}, {mn}",
                  f"v_exp_f32 {al}, {t0}",
                  f"v_cmp_eq_f32 vcc, {NEG_INF}, {mn}",
                  f"v_cndmask_b32_e64 {al}, {al}, 1.0, vcc",          # alpha = 1 if m_new = -inf
                  f"v_cndmask_b32_e64 {mm}, {mn}, 0, vcc",            # m used for P: 0 if -inf
                  f"v_mov_b32 v{M + qb}, {mn}",
                  f"v_mul_f32 v{L + qb}, v{L + qb}, {al}"]
        # O^T of this row block *= alpha, four values at a time
        vals = [(db, v) for db in range(4) for v in range(16)]
        for k in range(0, 64, 4):
            grp = vals[k:k + 4]
            tmps = [f"v{136 + i}" for i in range(4)]   # v136..v139
            lines += [f"v_accvgpr_read_b32 {tmps[i]}, {o_elem(db, qb, v)}" for i, (db, v) in enumerate(grp)]
            lines += [f"v_mul_f32 {tmps[i]}, {tmps[i]}, {al}" for i in range(4)]
            lines += [f"v_accvgpr_write_b32 {o_elem(db, qb, v)}, {tmps[i]}" for i, (db, v) in enumerate(grp)]
        # P of the tile at the new m, and its sums
        s0, s1 = "v140", "v141"
        lines += [f"v_mov_b32 {s0}, 0", f"v_mov_b32 {s1}, 0"]
        lines += softmax_ops(pc, masked, qbs=(qb,), mreg=lambda _q: mm,
                             sums=lambda _q, i: s0 if i == 0 else s1)
        lines += ["s_nop 3", f"v_add_f32 v{L + qb}, v{L + qb}, {s0}", f"v_add_f32 v{L + qb}, v{L + qb}, {s1}"]
    lines.append("s_nop 3")
    return lines


def init_block():
    """O = 0, S = 0, P = 0 (P(-1) = 0 is read by the first PV), m = -inf, sums, masks, l = 0."""
    lines = [f"v_accvgpr_write_b32 a{i}, 0" for i in range(128)]
    lines += [f"v_mov_b32 v{i}, 0" for i in range(128)]
    lines += [f"v_mov_b32 v{M}, {NEG_INF}", f"v_mov_b32 v{M + 1}, {NEG_INF}"]
    lines += [f"v_mov_b32 v{i}, 0" for i in list(range(TS, CMASK + 2)) + [L, L + 1]]
    return lines


def pv_only_block(pp):
    return stream(v_reads(), pp, []) + ["s_nop 11"]


def check_hazards(lines):
    """An MFMA result is not read by a VALU op within 12 instructions; a register an MFMA reads
    is not overwritten by an LDS read within 12 instructions; an exponential's result is not
    read by the next instruction."""
    last_write = {}
    last_exp = {}
    last_mfma_read = {}
    last_dot = {}
    for idx, l in enumerate(lines):
        op = l.split()[0] if l.split() else ""
        if op.startswith("v_mfma"):
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


KOFF, VOFF, SLOTL = 230, 234, 238
KTILE = 16384                                    # bytes of a K (or V^T) tile in LDS


def wait_loads(tag):
    """Own loads of K(t), V(t-1) in: vmcnt(nlprev), nlprev in {0, 4, 8}."""
    return ["s_cmp_eq_u32 %[nlprev], 8", f"s_cbranch_scc1 .Lw64_w8{tag}_%=",
            "s_cmp_eq_u32 %[nlprev], 4", f"s_cbranch_scc1 .Lw64_w4{tag}_%=",
            "s_waitcnt vmcnt(0)", f"s_branch .Lw64_wd{tag}_%=",
            f".Lw64_w8{tag}_%=:", "s_waitcnt vmcnt(8)", f"s_branch .Lw64_wd{tag}_%=",
            f".Lw64_w4{tag}_%=:", "s_waitcnt vmcnt(4)",
            f".Lw64_wd{tag}_%=:"]


def dma(kind, tag):
    """Load the next K (t+2) or V^T (t+1) tile if it exists: advance the cursor, offset of the
    tile inside the (layer, head) block, four 1 KB loads of this wave's share into ring slot
    (offset kl / vl, advanced first), lane offsets koff / voff."""
    f, k, blk, lo, off, ahead, mbase, colb = (("kf", "kk", "kblk", "kl", KOFF, 2, "mk", 14) if kind == "K"
                                              else ("vf", "vk", "vblk", "vl", VOFF, 1, "mv", 7))
    skip = f".Lw64_no{kind}{tag}_%="
    lines = [f"s_add_u32 %[x], %[t], {ahead}", "s_cmp_lt_u32 %[x], %[n]", f"s_cbranch_scc0 {skip}",
             f"s_add_u32 %[{k}], %[{k}], 1", f"s_cmp_eq_u32 %[{k}], %[tpf]",
             f"s_cselect_b32 %[{k}], 0, %[{k}]", f"s_addc_u32 %[{f}], %[{f}], 0",
             f"v_readlane_b32 %[x], v{SLOTL}, %[{f}]",
             "s_mul_i32 %[x], %[x], %[slotb]",
             f"s_lshl_b32 %[y], %[{k}], {colb}",       # tile within the frame: 16 KB of K rows / 128 B of V^T columns
             "s_add_u32 %[x], %[x], %[y]",
             f"s_add_u32 %[{lo}], %[{lo}], {KTILE}", f"s_cmp_eq_u32 %[{lo}], {3 * KTILE}",
             f"s_cselect_b32 %[{lo}], 0, %[{lo}]",
             f"s_add_u32 m0, %[{mbase}], %[{lo}]"]
    for i in range(4):
        lines += [f"v_add_u32 v{128 + 4 * (kind == 'V') + i}, %[x], v{off + i}"]
    for i in range(4):
        if i:
            lines.append("s_add_u32 m0, m0, 1024")
        lines.append(f"global_load_lds_dwordx4 v{128 + 4 * (kind == 'V') + i}, %[{blk}]")
    lines += ["s_add_u32 %[nl], %[nl], 4", f"{skip}:"]
    return lines


def iteration(pp, tag):
    """Iteration t < n (P buffer pp read by PV(t-1), P(t) written into 1 - pp)."""
    pc = 1 - pp
    lines = wait_loads(tag) + ["s_barrier", "s_mov_b32 %[nl], 0"]
    lines += dma("K", tag) + dma("V", tag)
    lines += ["s_mov_b32 %[nlprev], %[nl]",
              # tile t: valid keys, own frame index, masked?
              "s_lshl_b32 %[x], %[sk], 6", "s_sub_i32 %[nvalid], %[N], %[x]",
              "s_min_i32 %[nvalid], %[nvalid], 64",
              "s_sub_i32 %[tk], %[sf], %[nshared]",
              "s_cmp_lt_i32 %[nvalid], 64", "s_cselect_b32 %[mflag], 1, 0",
              "s_cmp_gt_i32 %[tk], %[tqw]", "s_cselect_b32 %[x], 1, 0",
              "s_or_b32 %[mflag], %[mflag], %[x]",
              # LDS read address steps to K(t+1), V(t)
              f"s_movk_i32 %[kstep], {KTILE}", f"s_movk_i32 %[x], {hex((-2 * KTILE) & 0xffff)}",
              "s_cmp_eq_u32 %[krd], 2", "s_cselect_b32 %[kstep], %[x], %[kstep]",
              "s_add_u32 %[krd], %[krd], 1", "s_cmp_eq_u32 %[krd], 3", "s_cselect_b32 %[krd], 0, %[krd]",
              f"s_movk_i32 %[vstep], {KTILE}",
              "s_cmp_eq_u32 %[vrd], 2", "s_cselect_b32 %[vstep], %[x], %[vstep]",
              "s_add_u32 %[vrd], %[vrd], 1", "s_cmp_eq_u32 %[vrd], 3", "s_cselect_b32 %[vrd], 0, %[vrd]",
              "s_cmp_eq_u32 %[mflag], 0", f"s_cbranch_scc0 .Lw64_m{tag}_%="]
    lines += tile_block(pp, False, tag + "u")
    lines += [f"s_branch .Lw64_td{tag}_%=", f".Lw64_m{tag}_%=:"]
    lines += tile_block(pp, True, tag + "m")
    lines += [f".Lw64_td{tag}_%=:",
              "s_cmp_eq_u64 %[trig], 0", f"s_cbranch_scc1 .Lw64_nr{tag}_%=",
              "s_cmp_eq_u32 %[mflag], 0", f"s_cbranch_scc1 .Lw64_ru{tag}_%="]
    lines += rare_block(pc, True)
    lines += [f"s_branch .Lw64_nr{tag}_%=", f".Lw64_ru{tag}_%=:"]
    lines += rare_block(pc, False)
    lines += [f".Lw64_nr{tag}_%=:",
              # next tile of the softmax walk
              "s_add_u32 %[x], %[t], 1", "s_cmp_lt_u32 %[x], %[n]", f"s_cbranch_scc0 .Lw64_ns{tag}_%=",
              "s_add_u32 %[sk], %[sk], 1", "s_cmp_eq_u32 %[sk], %[tpf]",
              "s_cselect_b32 %[sk], 0, %[sk]", "s_addc_u32 %[sf], %[sf], 0",
              f".Lw64_ns{tag}_%=:",
              "s_add_u32 %[t], %[t], 1"]
    return lines


def loop_program():
    """The whole tile loop: iterations t = 0 .. n-1 (two per pass, P buffer parity fixed),
    then the last PV.  m0 is saved and restored."""
    lines = ["s_mov_b32 %[m0save], m0"] + init_block()
    lines += [".Lw64_loop_%=:"] + iteration(1, "a")
    lines += ["s_cmp_lt_u32 %[t], %[n]", "s_cbranch_scc0 .Lw64_end_%="]
    lines += iteration(0, "b")
    lines += ["s_cmp_lt_u32 %[t], %[n]", "s_cbranch_scc1 .Lw64_loop_%=",
              ".Lw64_end_%=:"] + wait_loads("z") + ["s_barrier",
              "s_bitcmp1_b32 %[n], 0", "s_cbranch_scc0 .Lw64_pv1_%="]
    lines += pv_only_block(0) + ["s_branch .Lw64_fin_%=", ".Lw64_pv1_%=:"] + pv_only_block(1)
    lines += [".Lw64_fin_%=:", "s_mov_b32 m0, %[m0save]"]
    return lines


def emit(name, lines):
    check_hazards([l for l in lines if not l.startswith(".L")])
    body = " \\\n".join(f'  "{l}\\n\\t"' for l in lines)
    return f"#define {name} \\\n{body}\n"


def main():
    out = ["// Generated by gen_attn_w64.py; do not edit.  The tile loop of the 64-row attention",
           "// kernel as one asm program (register plan, blocks and hazard rules in the generator).", ""]
    out.append(emit("SDV2_W64_LOOP", loop_program()))
    sys.stdout.write("\n".join(out))


if __name__ == "__main__":
    main()
