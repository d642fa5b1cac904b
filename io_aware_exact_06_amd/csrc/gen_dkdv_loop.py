"""Generate attn_dkdv_loop.inc: the dK/dV kernel's walk over unmasked query
tiles (d = 128, one wave per SIMD), scheduled by hand as one inline-assembly
statement per input type.

What the loop computes is exactly the C++ tile of attn_bwd.hip (the hotdry
blog's section "4. 重计算（Recomputation）策略": S and dP are rebuilt from
Q, K, dO, V and the stored row statistics, then P = exp(scale s - lse),
dS = P o (dP - D), dV^T += dO^T P, dK^T += Q^T dS).  Every instruction, its
operands and the order of every accumulation are the C++ tile's, so the
results are bitwise equal; the schedule differs.

Per wave (32 keys) the query rows come in blocks k of 32, two per 64-row tile.
Iteration k of the loop issues
  run 1: the 16 dV / dK MFMAs of block k-1 (operands read transposed from its
         tile), then, for odd k, the tile boundary (DMA wait, the next tile's
         row statistics into LDS, barrier, the DMA of the tile after it);
  run 2: the 16 S / dP MFMAs of block k+1 (operands read from its tile);
and spreads the vector work of block k (P, dS and their packing, 64
instructions with 16 exponentials) over both runs.  The C++ tile issues S, dP
of a block alone and then its vector work beside the previous block's dV, dK:
with one wave per SIMD nothing else fills the matrix cores while it waits.
LDS operands go into a ring of 16 four-register AGPR slots and are read seven
MFMAs ahead (at most 15 LDS instructions in flight, the counter's range); the row statistics of block k+1 are read during block k.

Register map (physical; 512 per lane at one wave per SIMD):
  a0..a63     dV^T accumulators      a64..a127  dK^T accumulators
  a128..a159  K fragments            a160..a191 V fragments
  a192..a255  LDS operand ring (16 slots)
  v0..v31     S, dP of even blocks   v32..v63   S, dP of odd blocks
  v64..v79    packed P, dS of even blocks (B operands)   v80..v95 of odd blocks
  v96..v127   lse*log2e and -D rows of even blocks       v128..v159 of odd blocks
              (the -D rows are the initial accumulators of dP: the products leave dP - D)
  v160, v161  the next tile's lse and -D rows as loaded by wave 0 (lse is scaled by
              log2(e) when it is stored to LDS, as in the C++ boundary)
SGPR pairs s[80:81], s[82:83], s[84:85], s[86:87]: DMA sources of the next Q
and dO tile, and the next tile's lse and D rows.

Wait states are padded by the same checker as the forward loop's
(gen_fwd_loop.Stream); LDS results are waited for with lgkmcnt counts
computed from the order of every LDS instruction issued.

Run: python gen_dkdv_loop.py <output.inc>   (the build runs it before compiling)
"""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from gen_fwd_loop import TYPES, Stream, vr  # noqa: E402

HEAD_DIMS = (128,)
AHEAD = 7            # MFMAs whose LDS operands are read ahead (ring of 16 slots; at most 15 reads in flight)
KLOG2E = "0x3fb8aa3b"

ACC_DV, ACC_DK, KF, VF, RING = 0, 64, 128, 160, 192
SDP = (0, 32)        # S at +0, dP at +16 of a block set
PK = (64, 80)        # packed P at +0 (two u32x4), dS at +8
STAT = (96, 128)     # lse*log2e rows at +0 (four f32x4), D rows at +16
STL, STD = 160, 161
TMP = 162
NSLOT = 16
# the read issued after MFMA j fills slot (j + AHEAD) % NSLOT, which must not be
# the slot of MFMA j or of any MFMA still waiting for its operand
assert AHEAD < NSLOT


def ar(a, n=1):
    return "a%d" % a if n == 1 else "a[%d:%d]" % (a, a + n - 1)


class LdsStream(Stream):
    """Stream plus the order of the LDS instructions in flight, so that every
    read of an LDS result is preceded by the right lgkmcnt wait."""

    def __init__(self):
        super().__init__()
        self.lds = []  # destination register sets of the LDS instructions in flight, oldest first

    def _wait_to(self, k):
        """s_waitcnt lgkmcnt(k): LDS instructions complete in order, so all but the k youngest have."""
        self.raw("s_waitcnt lgkmcnt(%d)" % k, 1)
        self.lds = self.lds[len(self.lds) - k:] if k else []

    def lds_op(self, text, dst=()):
        # the counter has 4 bits: never more than 15 LDS instructions in flight
        if len(self.lds) >= 15:
            self._wait_to(14)
        self.ins(text, "ds", [], list(dst))
        self.lds.append(set(dst))

    def lds_wait(self, regs):
        regs = set(regs)
        last = -1
        for i, d in enumerate(self.lds):
            if d & regs:
                last = i
        if last >= 0:
            self._wait_to(len(self.lds) - 1 - last)

    def lds_drain(self):
        if self.lds:
            self.raw("s_waitcnt lgkmcnt(0)", 1)
            self.lds = []


def generate(T, D):
    mfma, cvt, _, _ = TYPES[T]
    KS, DB, CG = D // 16, D // 32, D // 32
    TBB = 64 * D * 2                     # bytes of one 64-row tile
    PER_WAVE = (64 // 16) * CG // 4      # DMA instructions per wave and tensor
    HI = 3 * TBB                         # byte offset of the second set of base registers
    S = LdsStream()
    labels = [0]

    def label(name):
        labels[0] += 1
        return "L_%s_%d_%%=" % (name, labels[0])

    def base(tile_off, kind):
        """Base register (operand name) and immediate for a byte offset into smem."""
        if tile_off < HI:
            return "%%[%s_lo" % kind, tile_off
        return "%%[%s_hi" % kind, tile_off - HI

    def q_tile(b):
        return 2 * b * TBB

    def do_tile(b):
        return (2 * b + 1) * TBB

    # ---------------------------------------------------------------- the parts
    def a_mfmas(b, qb, s_set):
        """S = Q K^T (even i) and dP = dO V^T (odd i) of block qb of the tile in buffer b."""
        out = []
        for i in range(2 * KS):
            tile = do_tile(b) if i & 1 else q_tile(b)
            off = tile + (2 * qb * CG + (i >> 1) // 2) * 1024
            reg, imm = base(off, "f")
            reads = [("ds_read_b128", "%s%d]" % (reg, (i >> 1) & 1), imm, 4, 0)]
            dst = SDP[s_set] + (16 if i & 1 else 0)
            bop = (VF if i & 1 else KF) + 4 * (i >> 1)
            # S starts from 0, dP from the -D rows of the block (so it ends as dP - D)
            c0 = STAT[s_set] + 16 if i == 1 else None
            out.append(dict(reads=reads, dst=dst, acc_agpr=False, b=ar(bop, 4), b_regs=(), first=(i >> 1) == 0,
                            c0=c0))
        return out

    def b_mfmas(b, qp, p_set):
        """dV^T += dO^T P (even i) and dK^T += Q^T dS (odd i) of block qp of the tile in buffer b."""
        out = []
        for i in range(4 * DB):
            tile = q_tile(b) if i & 1 else do_tile(b)
            off = tile + ((2 * qp + ((i >> 1) & 1)) * CG + (i >> 2)) * 1024
            reg, imm = base(off, "t")
            reads = [("ds_read_b64_tr_b16", "%s0]" % reg, imm, 2, 0), ("ds_read_b64_tr_b16", "%s1]" % reg, imm, 2, 2)]
            dst = (ACC_DK if i & 1 else ACC_DV) + 16 * (i >> 2)
            bb = PK[p_set] + (8 if i & 1 else 0) + 4 * ((i >> 1) & 1)
            out.append(dict(reads=reads, dst=dst, acc_agpr=True, b=vr(bb, 4), b_regs=tuple(range(bb, bb + 4)),
                            first=False))
        return out

    def v_ops(s_set, p_set):
        """P = exp2(s c - lse log2e), dS = P (dP - D) (the dP accumulator already holds
        dP - D), packed as B operands (the C++ element order)."""
        sb, dpb = SDP[s_set], SDP[s_set] + 16
        lb = STAT[s_set]
        pb, dsb = PK[p_set], PK[p_set] + 8
        ops = []
        for e in range(16):
            g, r = e >> 2, e & 3
            l = lb + 4 * g + r
            ops.append(("v_fma_f32 %s, %s, %%[c], -%s" % (vr(sb + e), vr(sb + e), vr(l)), "valu", [sb + e, l], [sb + e]))
            ops.append(("v_exp_f32 %s, %s" % (vr(sb + e), vr(sb + e)), "trans", [sb + e], [sb + e]))
            ops.append(("v_mul_f32 %s, %s, %s" % (vr(dpb + e), vr(sb + e), vr(dpb + e)), "valu", [sb + e, dpb + e], [dpb + e]))
            if e & 1:
                q = (e & 7) >> 1
                t = e >> 3
                ops.append(("%s %s, %s, %s" % (cvt, vr(pb + 4 * t + q), vr(sb + e - 1), vr(sb + e)), "valu",
                            [sb + e - 1, sb + e], [pb + 4 * t + q]))
                ops.append(("%s %s, %s, %s" % (cvt, vr(dsb + 4 * t + q), vr(dpb + e - 1), vr(dpb + e)), "valu",
                            [dpb + e - 1, dpb + e], [dsb + 4 * t + q]))
        return ops

    def stat_reads(b, qc, s_set):
        """lse*log2e and D of the 32 rows of block qc, from the statistics of buffer b (8 x 128-bit)."""
        out = []
        for which in (0, 1):
            for g in range(4):
                off = ((b * 2 + which) * 64 + 32 * qc + 8 * g) * 4
                dst = STAT[s_set] + 16 * which + 4 * g
                out.append(("ds_read_b128 %s, %%[st] offset:%d" % (vr(dst, 4), off), list(range(dst, dst + 4))))
        return out

    # ---------------------------------------------------------------- emission helpers
    slot = [0]       # next ring slot

    def run_mfmas(mlist, vops, vquota, extra_reads=None, after=None, pre_reads=()):
        """Issue the MFMAs of mlist with their LDS reads AHEAD slots ahead and vquota[j]
        vector ops after MFMA j; extra_reads (LDS reads into other registers) are
        issued after the second MFMA, after[j] (scalar and memory instructions)
        right after MFMA j.  Returns the remaining vector ops."""
        after = after or {}
        n = len(mlist)
        slots = []
        for _ in range(n):
            slots.append(slot[0])
            slot[0] = (slot[0] + 1) % NSLOT

        def issue(j):
            if j < n:
                sl = RING + 4 * slots[j]
                for (op, addr, imm, nreg, half) in mlist[j]["reads"]:
                    dst = sl + half
                    S.lds_op("%s %s, %s offset:%d" % (op, ar(dst, nreg), addr, imm),
                             ["a%d" % r for r in range(dst, dst + nreg)])
        for (t, dst) in pre_reads:
            S.lds_op(t, dst)
        ahead = min(AHEAD, n)
        for j in range(ahead):
            issue(j)
        pending = list(extra_reads or [])
        for j, M in enumerate(mlist):
            emit_mfma(M, slots[j])
            issue(j + ahead)
            for fn in after.get(j, []):
                fn()
            if j == 1 and pending:
                for (t, dst) in pending:
                    S.lds_op(t, dst)
                pending = []
            for _ in range(vquota[j]):
                if vops:
                    emit_v(vops.pop(0))
        for (t, dst) in pending:
            S.lds_op(t, dst)
        return vops

    def emit_mfma(M, slot_index):
        sl = RING + 4 * slot_index
        c0 = M.get("c0")
        S.lds_wait(["a%d" % r for r in range(sl, sl + 4)] + (list(range(c0, c0 + 16)) if c0 is not None else []))
        reads = list(M["b_regs"]) + ([] if M["first"] or M["acc_agpr"] else list(range(M["dst"], M["dst"] + 16)))
        if c0 is not None:
            reads += list(range(c0, c0 + 16))
        dn = ar(M["dst"], 16) if M["acc_agpr"] else vr(M["dst"], 16)
        c = (vr(c0, 16) if c0 is not None else "0") if M["first"] else dn
        S.ins("%s %s, %s, %s, %s" % (mfma, dn, ar(sl, 4), M["b"], c), "mfma", reads,
              [] if M["acc_agpr"] else list(range(M["dst"], M["dst"] + 16)),
              acc=None if M["acc_agpr"] else tuple(range(M["dst"], M["dst"] + 16)))

    def emit_v(op):
        t, k, r, w = op
        S.lds_wait(r)
        S.ins(t, k, r, w)

    def quotas(total, n):
        out, done = [], 0
        for j in range(n):
            want = round((j + 1) * total / n)
            out.append(want - done)
            done = want
        return out

    def boundary(bc, bn, bpv):
        """Tile boundary: the next tile (buffer bn) has landed; its statistics go
        to LDS; the tile after it goes into buffer bpv."""
        skip_st, skip_ld = label("nostat"), label("noload")
        S.lds_drain()
        S.raw("s_waitcnt vmcnt(0)", 1)
        S.raw("s_cmp_lg_u32 %[w], 0", 1)
        S.raw("s_cbranch_scc1 %s" % skip_st, 1)
        S.raw("v_mul_f32 %s, %s, %s" % (vr(STL), KLOG2E, vr(STL)), 1)
        S.nop(1)
        S.raw("ds_write_b32 %%[sw], %s offset:%d" % (vr(STL), (bn * 2 + 0) * 64 * 4), 1)
        S.raw("ds_write_b32 %%[sw], %s offset:%d" % (vr(STD), (bn * 2 + 1) * 64 * 4), 1)
        S.raw("s_waitcnt lgkmcnt(0)", 1)
        S.raw("%s:" % skip_st)
        S.raw("s_barrier", 1)

    def loads(bpv):
        """The loads of the tile after the next, issued one by one between the
        MFMAs that follow the boundary (bunched, they stall at issue): {MFMA
        index: [emitters]}.  Buffer bpv is free once every wave has passed the
        boundary's barrier."""
        skip_ld = label("noload")
        out = {}

        def dma(mreg, src, i):
            def f():
                S.raw("s_add_u32 m0, %s, %d" % (mreg, 4096 * i), 1)
                S.nop(1)
                S.raw("global_load_lds_dwordx4 %%[g%d], %s" % (i, src), 1)
            return f

        def stats():
            S.raw("s_cmp_lg_u32 %[w], 0", 1)
            S.raw("s_cbranch_scc1 %s" % skip_ld, 1)
            S.raw("global_load_dword %s, %%[so], s[84:85]" % vr(STL), 1)
            S.raw("global_load_dword %s, %%[so], s[86:87]" % vr(STD), 1)
            S.raw("%s:" % skip_ld)

        def advance():
            for pair, step in (("80", TBB), ("82", TBB), ("84", 256), ("86", 256)):
                lo = int(pair)
                S.raw("s_add_u32 s%d, s%d, %d" % (lo, lo, step), 1)
                S.raw("s_addc_u32 s%d, s%d, 0" % (lo + 1, lo + 1), 1)
        seq = []
        for i in range(PER_WAVE):
            seq.append(dma("%%[mq%d]" % bpv, "s[80:81]", i))
            seq.append(dma("%%[md%d]" % bpv, "s[82:83]", i))
        out[0] = [stats]
        for k, f in enumerate(seq):
            out.setdefault(2 * k + 1, []).append(f)
        out[2 * len(seq) - 1].append(advance)  # after the last DMA
        return out

    # ---------------------------------------------------------------- the statement
    S.nop(24)
    # entry: S, dP of block 0 of the first tile (buffer = phase), its statistics
    exits = []
    for ph in range(3):
        S.raw("s_cmp_eq_u32 %%[phase], %d" % ph)
        S.raw("s_cbranch_scc1 L_pro%d_%%=" % ph)
    S.raw("s_branch L_pro0_%=")
    for ph in range(3):
        S.raw("L_pro%d_%%=:" % ph)
        S.last, S.lds = {}, []
        slot[0] = 0
        for (t, dst) in stat_reads(ph, 0, 0):
            S.lds_op(t, dst)
        run_mfmas(a_mfmas(ph, 0, 0), [], [0] * (2 * KS))
        S.lds_drain()
        S.raw("s_branch L_t%d_%%=" % ph)
    # the tile loop, unrolled over the three buffer rotations
    for ph in range(3):
        bc, bn, bpv = ph, (ph + 1) % 3, (ph + 2) % 3
        S.raw("L_t%d_%%=:" % ph)
        S.last, S.lds = {}, []
        # entered from the prologue or the previous tile: S, dP of block 0 were
        # just written by MFMAs and the packed P, dS of block 1 by the VALU
        for r in range(SDP[0], SDP[0] + 32):
            S.last[r] = (S.pos - 1, "mfma", None)
        for r in range(PK[1], PK[1] + 16):
            S.last[r] = (S.pos - 1, "valu", None)
        slot[0] = 0
        # iteration 2t: B(block 1 of the previous tile, buffer bpv, packed set 1),
        # A(block 1 of this tile, buffer bc, S set 1); V(block 0: S set 0 -> packed set 0)
        v0 = v_ops(0, 0)
        ml = b_mfmas(bpv, 1, 1) + a_mfmas(bc, 1, 1)
        rest = run_mfmas(ml, v0, quotas(len(v0), len(ml)), extra_reads=stat_reads(bc, 1, 1))
        for op in rest:
            emit_v(op)
        # iteration 2t+1: B(block 0, buffer bc, packed set 0), boundary, A(block 0 of
        # the next tile, buffer bn, S set 0); V(block 1: S set 1 -> packed set 1)
        v1 = v_ops(1, 1)
        half = len(v1) // 2
        rest = run_mfmas(b_mfmas(bc, 0, 0), v1, quotas(half, 4 * DB))
        boundary(bc, bn, bpv)
        S.raw("s_sub_u32 %[n], %[n], 1", 1)
        S.raw("s_cmp_eq_u32 %[n], 0", 1)
        ex = label("exit")
        S.raw("s_cbranch_scc1 %s" % ex, 1)
        exits.append((ex, list(rest), bpv))
        # the -D rows first: the run's second MFMA starts from them
        st_rd = stat_reads(bn, 0, 0)
        rest = run_mfmas(a_mfmas(bn, 0, 0), rest, quotas(len(rest), 2 * KS), pre_reads=st_rd[4:], extra_reads=st_rd[:4],
                         after=loads(bpv))
        for op in rest:
            emit_v(op)
        S.lds_drain()
        S.raw("s_branch L_t%d_%%=" % ((ph + 1) % 3))
    # exits: the rest of block 1's vector work, then wait for every load of the statement
    for ex, rest, bpv in exits:
        # the walk ends at this boundary: the loads of the tile after the next,
        # then the rest of block 1's vector work
        S.raw("%s:" % ex)
        S.last, S.lds = {}, []
        for j, fns in sorted(loads(bpv).items()):
            for fn in fns:
                fn()
        for op in rest:
            emit_v(op)
        S.raw("s_branch L_done_%=")
    S.raw("L_done_%=:")
    S.lds_drain()
    # the statistics loads (issued before the 2 x PER_WAVE tile DMAs of the exit
    # block) must land inside the statement; the DMA may stay in flight: the
    # C++ boundary waits for it
    S.raw("s_waitcnt vmcnt(%d)" % (2 * PER_WAVE))
    S.nop(24)
    return S.out


SIGNATURE = ("f32x16 (&dv)[%(DB)s], f32x16 (&dk)[%(DB)s], const u32x4 (&kf)[%(KS)s], const u32x4 (&vf)[%(KS)s], "
             "u32x4 (&bp1)[2], u32x4 (&bds1)[2], float& stl, float& std_, const uint32_t (&f)[4], "
             "const uint32_t (&t)[4], uint32_t st, uint32_t sw, const uint32_t (&g)[4], uint32_t so, float c, "
             "uint32_t w, uint32_t phase, const uint32_t (&mq)[3], const uint32_t (&md)[3], uint64_t qsrc, "
             "uint64_t dosrc, uint64_t lsrc, uint64_t dsrc, uint32_t n")


def function(T, D):
    KS, DB = D // 16, D // 32
    PER_WAVE = (64 // 16) * (D // 32) // 4
    body = "\\n\\t".join(generate(T, D))
    outs = ['"+{a[%d:%d]}"(dv[%d])' % (ACC_DV + 16 * i, ACC_DV + 16 * i + 15, i) for i in range(DB)]
    outs += ['"+{a[%d:%d]}"(dk[%d])' % (ACC_DK + 16 * i, ACC_DK + 16 * i + 15, i) for i in range(DB)]
    outs += ['"+{v[%d:%d]}"(bp1[%d])' % (PK[1] + 4 * i, PK[1] + 4 * i + 3, i) for i in range(2)]
    outs += ['"+{v[%d:%d]}"(bds1[%d])' % (PK[1] + 8 + 4 * i, PK[1] + 8 + 4 * i + 3, i) for i in range(2)]
    outs += ['"+{v%d}"(stl)' % STL, '"+{v%d}"(std_)' % STD, '[n] "+s"(n)', '"+{s[80:81]}"(qsrc)',
             '"+{s[82:83]}"(dosrc)', '"+{s[84:85]}"(lsrc)', '"+{s[86:87]}"(dsrc)']
    ins = ['"{a[%d:%d]}"(kf[%d])' % (KF + 4 * i, KF + 4 * i + 3, i) for i in range(KS)]
    ins += ['"{a[%d:%d]}"(vf[%d])' % (VF + 4 * i, VF + 4 * i + 3, i) for i in range(KS)]
    ins += ['[f_lo0] "v"(f[0])', '[f_lo1] "v"(f[1])', '[f_hi0] "v"(f[2])', '[f_hi1] "v"(f[3])',
            '[t_lo0] "v"(t[0])', '[t_lo1] "v"(t[1])', '[t_hi0] "v"(t[2])', '[t_hi1] "v"(t[3])',
            '[st] "v"(st)', '[sw] "v"(sw)', '[so] "v"(so)']
    ins += ['[g%d] "v"(g[%d])' % (i, i) for i in range(PER_WAVE)]
    ins += ['[c] "s"(c)', '[w] "s"(w)', '[phase] "s"(phase)']
    ins += ['[mq%d] "s"(mq[%d])' % (i, i) for i in range(3)] + ['[md%d] "s"(md[%d])' % (i, i) for i in range(3)]
    vclob = [r for r in range(0, TMP + 1) if not (PK[1] <= r < PK[1] + 16) and r not in (STL, STD)]
    clobbers = ", ".join(['"v%d"' % r for r in vclob] + ['"a%d"' % r for r in range(RING, RING + 4 * NSLOT)])
    return "\n".join([
        "template <>",
        "__device__ inline void dkdv_unmasked_run<%s, %d>(%s) {" % (T, D, SIGNATURE % {"DB": DB, "KS": KS}),
        '    asm volatile("%s"' % body,
        "                 : " + ",\n                   ".join(outs),
        "                 : " + ",\n                   ".join(ins),
        '                 : %s, "vcc", "scc", "m0", "memory");' % clobbers,
        "}"])


HEADER = """// attn_dkdv_loop.inc -- generated by gen_dkdv_loop.py (run by the build); do not edit.
//
// dkdv_unmasked_run<T, D>: n consecutive unmasked query tiles of the dK/dV
// kernel's walk, as one inline-assembly statement.  On entry: the walk is at
// the start of a tile in ring buffer `phase` (landed, its statistics in LDS),
// the next tile's DMA is in flight and its lse and D rows are in stl / std_
// (wave 0; lse unscaled), bp1 / bds1 hold the packed P and dS of the previous tile's second
// block, and qsrc / dosrc / lsrc / dsrc point at the tile after the next
// (plus this wave's block offset).  On exit the walk is at the start of the
// tile after the last one, in the same state (the next tile's DMA in flight,
// its statistics landed).  f / t: LDS read addresses (two lane patterns, from the
// start of the tile ring and from three tiles further); st / sw: this lane's
// statistics read and write addresses; g: DMA lane offsets; so: this lane's
// statistics load offset; mq / md: DMA LDS destinations of the Q and dO tiles
// of the three buffers for this wave.
// n >= 1: the statement counts tiles down to zero, so a count of 0 would not end.
"""


def main(path):
    parts = [HEADER, "template <class T, int D>",
             "__device__ inline void dkdv_unmasked_run(%s);" % (SIGNATURE % {"DB": "D / 32", "KS": "D / 16"})]
    for T in ("BF16", "F16"):
        for D in HEAD_DIMS:
            parts.append(function(T, D))
    text = "\n".join(parts[:3]) + "\n\n" + "\n\n".join(parts[3:]) + "\n"
    old = open(path).read() if os.path.exists(path) else None
    if old != text:
        with open(path, "w") as fh:
            fh.write(text)


if __name__ == "__main__":
    main(sys.argv[1])
