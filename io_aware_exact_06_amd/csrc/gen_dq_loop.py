"""Generate attn_dq_loop.inc: the dQ kernel's walk over unmasked key tiles
(d = 64 and 128, two waves per SIMD), scheduled by hand as one
inline-assembly statement per input type and head size.

What the loop computes is exactly the C++ step of attn_bwd.hip (the hotdry
blog's section "4. 重计算（Recomputation）策略": S^T = K Q^T and dP^T = V dO^T
are rebuilt for the tile, P^T = exp(scale s - lse), dS^T = P^T o (dP^T - D),
dQ^T += K^T dS^T).  Every accumulator sees the C++ step's operands in the
C++ step's order, so the results are bitwise equal; only the interleave
differs.

Per tile and wave (64 keys, two key blocks kb of 32) the MFMAs (48 at d = 128,
24 at d = 64) run as S(kb0), S(kb1), dP(kb0), dP(kb1), dQ(kb0), dQ(kb1).  The vector work is split
by what it needs: the exponentials of kb (P) need only S(kb), the difference,
product and packing (dS) need dP(kb) as well; each piece goes between the
MFMAs from the first one that may issue it on, and the packed dS of kb is
complete before the first dQ(kb) MFMA.  The C++ step issues all 32 S, dP
MFMAs, then all the vector work, then dQ.  The dP accumulators start from -D
(16 registers filled once per statement), so dS needs no subtraction, as in
the C++ step.  The DMA instructions of the next tile (eight at d = 128, four
at d = 64) go one per two MFMAs (bunched, they stall at issue); one lane-offset
register serves all of them, the scalar source stepping 4096 bytes between
blocks.  LDS operands go through a ring of four four-register slots, read
three MFMAs ahead (the register file has no room for more at d = 128).

Register map at d = 128 (physical, two waves per SIMD: at most 256 VGPRs; at
d = 64 the same blocks, packed from v0 by regmap()):
  v0..v63    dQ^T accumulators (4 blocks of 32 head columns)
  v64..v95   S^T of the two key blocks     v96..v127  dP^T of the two key blocks
  v128..v159 Q^T fragments                 v160..v191 dO^T fragments
  v192..v207 packed dS^T of the two key blocks (B operands of the dQ MFMAs)
  v208..v223 LDS operand ring (4 slots)    v224, v225 lse*log2e and D of the row
  v226..v241 -D (the first C operand of each dP^T chain)
SGPR pairs s[80:81], s[82:83]: DMA sources of the next K and V tile.

Run: python gen_dq_loop.py <output.inc>   (the build runs it before compiling)
"""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from gen_dkdv_loop import LdsStream  # noqa: E402
from gen_fwd_loop import TYPES, vr  # noqa: E402

HEAD_DIMS = (64, 128)
NSLOT = 4            # the LDS operand ring (four registers a slot)
AHEAD = 3            # MFMAs whose operands are read ahead
# the read issued after MFMA j fills slot (j + AHEAD) % NSLOT, which must not be
# the slot of MFMA j or of any MFMA still waiting for its operand
assert AHEAD < NSLOT


def regmap(D):
    """Physical VGPR bases: dQ^T accumulators, S^T, dP^T, Q^T and dO^T fragments,
    packed dS^T, the LDS ring, lse*log2e, D and the 16 registers holding -D
    (d = 128: 0, 64, 96, 128, 160, 192, 208, 224, 225, 226; d = 64: 0, 32, 64,
    96, 112, 128, 144, 160, 161, 162)."""
    KS, DB = D // 16, D // 32
    acc = 0
    ss = acc + 16 * DB
    dp = ss + 32
    qf = dp + 32
    dof = qf + 4 * KS
    pk = dof + 4 * KS
    ring = pk + 16
    lse2 = ring + 4 * NSLOT
    return acc, ss, dp, qf, dof, pk, ring, lse2, lse2 + 1, lse2 + 2


def generate(T, D):
    mfma, cvt, _, _ = TYPES[T]
    KS, DB, CG = D // 16, D // 32, D // 32
    ACC, SS, DP, QF, DOF, PK, RING, LSE2, DQ, NEGD = regmap(D)
    TBB = 64 * D * 2
    PER_WAVE = (64 // 16) * CG // 4
    S = LdsStream()
    labels = [0]

    def label(name):
        labels[0] += 1
        return "L_%s_%d_%%=" % (name, labels[0])

    def frag_blk(rb, ks):
        return (2 * rb * CG + ks // 2) * 1024

    def tr_blk(rs, db):
        return (rs * CG + db) * 1024

    def mfmas(p):
        """The tile's MFMAs in issue order (K buffer p at p*TBB, V buffer p at (2+p)*TBB)."""
        out = []
        for kind in ("S0", "S1", "P0", "P1"):   # S(kb0), S(kb1), dP(kb0), dP(kb1)
            kb = int(kind[1])
            for ks in range(KS):
                tile = (p if kind[0] == "S" else 2 + p) * TBB
                off = tile + frag_blk(kb, ks)
                reads = [("ds_read_b128", "%%[f%d]" % (ks & 1), off, 4, 0)]
                dst = (SS if kind[0] == "S" else DP) + 16 * kb
                b = (QF if kind[0] == "S" else DOF) + 4 * ks
                # dP starts from -D (so it ends as dP - D)
                c0 = NEGD if (kind[0] == "P" and ks == 0) else None
                out.append(dict(reads=reads, dst=dst, b=b, first=ks == 0, c0=c0))
        for kb in range(2):                     # dQ(kb0), dQ(kb1): per db the C++ order kb, t
            for db in range(DB):
                for t in range(2):
                    off = p * TBB + tr_blk(2 * kb + t, db)
                    reads = [("ds_read_b64_tr_b16", "%[t0]", off, 2, 0), ("ds_read_b64_tr_b16", "%[t1]", off, 2, 2)]
                    out.append(dict(reads=reads, dst=ACC + 16 * db, b=PK + 8 * kb + 4 * t, first=False, c0=None))
        return out

    def p_ops(kb):
        s = SS + 16 * kb
        ops = []
        for e in range(16):
            ops.append(("v_fma_f32 %s, %s, %%[c], -%s" % (vr(s + e), vr(s + e), vr(LSE2)), "valu", [s + e], [s + e]))
            ops.append(("v_exp_f32 %s, %s" % (vr(s + e), vr(s + e)), "trans", [s + e], [s + e]))
        return ops

    def ds_ops(kb):
        s, dp, pk = SS + 16 * kb, DP + 16 * kb, PK + 8 * kb
        ops = []
        for e in range(16):  # the accumulator already holds dP - D
            ops.append(("v_mul_f32 %s, %s, %s" % (vr(dp + e), vr(s + e), vr(dp + e)), "valu", [s + e, dp + e], [dp + e]))
            if e & 1:
                d = pk + 4 * (e >> 3) + ((e & 7) >> 1)
                ops.append(("%s %s, %s, %s" % (cvt, vr(d), vr(dp + e - 1), vr(dp + e)), "valu", [dp + e - 1, dp + e], [d]))
        return ops

    def emit_mfma(M, slot_index):
        sl = RING + 4 * slot_index
        S.lds_wait(list(range(sl, sl + 4)))
        dst = list(range(M["dst"], M["dst"] + 16))
        reads = list(range(M["b"], M["b"] + 4)) + ([] if M["first"] else dst)
        c = "0" if M["first"] else vr(M["dst"], 16)
        if M["c0"] is not None:
            reads += list(range(M["c0"], M["c0"] + 16))
            c = vr(M["c0"], 16)
        S.ins("%s %s, %s, %s, %s" % (mfma, vr(M["dst"], 16), vr(sl, 4), vr(M["b"], 4), c), "mfma", reads, dst,
              acc=tuple(dst))

    def emit_v(op):
        t, k, r, w = op
        S.ins(t, k, r, w)

    def dma(p, i):
        """i < PER_WAVE: a block of the next K tile into K buffer 1-p; else of V."""
        kv = i >= PER_WAVE
        i %= PER_WAVE
        m0 = "%%[mv%d]" % (1 - p) if kv else "%%[mk%d]" % (1 - p)
        lo = 82 if kv else 80
        if i:  # the source of block i is 4096 bytes past block i - 1's (one lane-offset VGPR for all)
            S.raw("s_add_u32 s%d, s%d, 4096" % (lo, lo), 1)
            S.raw("s_addc_u32 s%d, s%d, 0" % (lo + 1, lo + 1), 1)
        S.raw("s_add_u32 m0, %s, %d" % (m0, 4096 * i), 1)
        S.nop(1)
        S.raw("global_load_lds_dwordx4 %%[g], s[%d:%d]" % (lo, lo + 1), 1)

    def tile(p):
        ML = mfmas(p)
        NM = len(ML)
        # The vector pieces in dependence order, each with the MFMA index after
        # which it may start (its inputs' last MFMA plus one: the hazard checker
        # pads what the pipeline does not cover) and the MFMA it must precede.
        n_s = KS  # MFMAs per S or dP block
        pieces = [(p_ops(0), n_s, None), (p_ops(1), 2 * n_s, None),
                  (ds_ops(0), 3 * n_s, 4 * n_s), (ds_ops(1), 4 * n_s, 4 * n_s + 2 * DB)]
        queue = [(op, earliest, deadline) for ops, earliest, deadline in pieces for op in ops]
        # spread by issue cost (an exponential holds the port about twice as
        # long as an add) evenly over the gaps from the first start to the last deadline
        cost = {"valu": 1.0, "trans": 2.0}
        total = sum(cost[op[1]] for op, _, _ in queue)
        first, last = pieces[0][1], pieces[-1][2] - 1
        slots = [j % NSLOT for j in range(NM)]

        def issue(j):
            if j < NM:
                sl = RING + 4 * slots[j]
                for (op, addr, imm, nreg, half) in ML[j]["reads"]:
                    dst = sl + half
                    S.lds_op("%s %s, %s offset:%d" % (op, vr(dst, nreg), addr, imm), list(range(dst, dst + nreg)))
        for j in range(AHEAD):
            issue(j)
        S.raw("s_setprio 1")
        done = 0.0
        for j, M in enumerate(ML):
            emit_mfma(M, slots[j])
            issue(j + AHEAD)
            if j < 2 * 2 * PER_WAVE and j % 2 == 1:
                dma(p, j // 2)
            # ops that must be done before the next MFMA, then the quota
            while queue and queue[0][2] is not None and queue[0][2] <= j + 1 and queue[0][1] <= j:
                done += cost[queue[0][0][1]]
                emit_v(queue.pop(0)[0])
            target = total * (j - first + 1) / (last - first + 1)
            while queue and done + 0.5 < target and queue[0][1] <= j:
                done += cost[queue[0][0][1]]
                emit_v(queue.pop(0)[0])
        while queue:
            emit_v(queue.pop(0)[0])
        S.raw("s_setprio 0")
        S.lds_drain()
        # the next tile has landed for this wave; every wave is done with this one
        S.raw("s_waitcnt vmcnt(0)", 1)
        S.raw("s_barrier", 1)
        back = 4096 * (PER_WAVE - 1)  # the DMA stepped the sources this far inside the tile
        S.raw("s_add_u32 s80, s80, %d" % (TBB - back))
        S.raw("s_addc_u32 s81, s81, 0")
        S.raw("s_add_u32 s82, s82, %d" % (TBB - back))
        S.raw("s_addc_u32 s83, s83, 0", 4)

    S.nop(24)
    # -D in all 16 elements (a sign flip, as the C++ negation)
    for e in range(16):
        S.ins("v_xor_b32 %s, 0x80000000, %s" % (vr(NEGD + e), vr(DQ)), "valu", [DQ], [NEGD + e])
    S.raw("s_cmp_eq_u32 %[par], 0")
    S.raw("s_cbranch_scc0 L_t1_%=")
    for p in (0, 1):
        S.raw("L_t%d_%%=:" % p)
        S.last, S.lds = {}, []
        tile(p)
        S.raw("s_sub_u32 %[n], %[n], 1", 1)
        S.raw("s_cmp_eq_u32 %[n], 0", 1)
        S.raw("s_cbranch_scc1 L_done_%=", 1)
    S.raw("s_branch L_t0_%=")
    S.raw("L_done_%=:")
    S.nop(24)
    return S.out


SIGNATURE = ("f32x16 (&dq)[%(DB)s], const u32x4 (&qf)[%(KS)s], const u32x4 (&dof)[%(KS)s], float lse2, float dqs, "
             "uint32_t f0, uint32_t f1, uint32_t t0, uint32_t t1, uint32_t g, float c, uint32_t par, "
             "uint32_t mk0, uint32_t mk1, uint32_t mv0, uint32_t mv1, uint64_t ksrc, uint64_t vsrc, uint32_t n")


def function(T, D):
    KS, DB = D // 16, D // 32
    ACC, SS, DP, QF, DOF, PK, RING, LSE2, DQ, NEGD = regmap(D)
    body = "\\n\\t".join(generate(T, D))
    outs = ['"+{v[%d:%d]}"(dq[%d])' % (ACC + 16 * i, ACC + 16 * i + 15, i) for i in range(DB)]
    outs += ['[n] "+s"(n)', '"+{s[80:81]}"(ksrc)', '"+{s[82:83]}"(vsrc)']
    ins = ['"{v[%d:%d]}"(qf[%d])' % (QF + 4 * i, QF + 4 * i + 3, i) for i in range(KS)]
    ins += ['"{v[%d:%d]}"(dof[%d])' % (DOF + 4 * i, DOF + 4 * i + 3, i) for i in range(KS)]
    ins += ['"{v%d}"(lse2)' % LSE2, '"{v%d}"(dqs)' % DQ]
    ins += ['[f0] "v"(f0)', '[f1] "v"(f1)', '[t0] "v"(t0)', '[t1] "v"(t1)']
    ins += ['[g] "v"(g)']
    ins += ['[c] "s"(c)', '[par] "s"(par)', '[mk0] "s"(mk0)', '[mk1] "s"(mk1)', '[mv0] "s"(mv0)', '[mv1] "s"(mv1)']
    negd = list(range(NEGD, NEGD + 16))
    clobbers = ", ".join('"v%d"' % r for r in list(range(SS, RING + 4 * NSLOT)) + negd
                         if not (QF <= r < DOF + 4 * KS))
    return "\n".join([
        "template <>",
        "__device__ inline void dq_unmasked_run<%s, %d>(%s) {" % (T, D, SIGNATURE % {"DB": DB, "KS": KS}),
        '    asm volatile("%s"' % body,
        "                 : " + ",\n                   ".join(outs),
        "                 : " + ",\n                   ".join(ins),
        '                 : %s, "vcc", "scc", "m0", "memory");' % clobbers,
        "}"])


HEADER = """// attn_dq_loop.inc -- generated by gen_dq_loop.py (run by the build); do not edit.
//
// dq_unmasked_run<T, D>: n consecutive unmasked key tiles of the dQ kernel's
// walk, starting at a tile in K/V buffer par, as one inline-assembly
// statement.  On entry the tile has landed in both buffers of parity par and
// nothing is in flight; ksrc / vsrc point at the next K and V tile (plus this
// wave's block offset).  Each tile loads the next into the other buffers,
// computes S^T, dP^T, P^T, dS^T and dQ^T += K^T dS^T, waits for the load and
// ends on a barrier, as the C++ step does.  f0 / f1 / t0 / t1: LDS read
// addresses (buffer 0); g: this lane's DMA offset within a block; mk / mv: DMA LDS destinations of
// the K and V buffers for this wave; lse2 = lse * log2(e) and dqs = D of this
// lane's query row; c = scale * log2(e).
// n >= 1: the statement counts tiles down to zero, so a count of 0 would not end.
"""


def main(path):
    parts = [HEADER, "template <class T, int D>",
             "__device__ inline void dq_unmasked_run(%s);" % (SIGNATURE % {"DB": "D / 32", "KS": "D / 16"})]
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
