"""Generate attn_fwd_loop.inc: the forward kernel's loop over unmasked key
tiles, scheduled by hand as one inline-assembly statement per input type.

What the loop computes is exactly the C++ step of attn_fwd.hip for a tile
that every row of the work group sees in full (the online softmax of the
hotdry blog, section "3. 在线softmax算法": raise the running maximum, rescale
the running sums and the partial output when it grew by more than 2^8 in
exp2 units, add the tile's exponentials and their weighted values).  The
instructions, their operands and the order of every floating-point
accumulation are the C++ step's, so the two paths give bitwise-equal results;
only the interleave differs:

* Per wave and tile (d = 128): 16 MFMAs for the scores of the next tile,
  16 for P.V of this tile, 48 LDS reads, 32 exponentials and about 120 other
  vector instructions.  The generator spreads the vector work evenly between
  the MFMAs (the C++ loop's compiler schedule bunches it), issues each LDS
  operand read six MFMAs ahead through a ring of eight 4-register slots, and
  issues the eight DMA instructions of the tile loads right after the step
  barrier.
* The maximum of the next tile's scores (and the lazy-rescale test) runs under
  the last P.V MFMAs of this step instead of at the start of the next one; the
  rescale itself (O, l, lh times alpha) is applied at the start of the next
  step, before anything adds to them.
* Rare paths (a rescale, a raised maximum) are branched to out of line.

gfx950 wait states that the hardware does not enforce are inserted by a small
checker over the emitted stream (conservative counts, one per instruction,
s_nop n counting n + 1): a VALU result read by an MFMA (2), an MFMA result
read by any other instruction (19, the 16-pass figure plus 3), a
transcendental result read by the VALU (1), a dot2c result read by anything
but the same dot2c accumulating into it (3); VALU-written lane masks and the
permlane swap get the nops the compiler itself emits around them.

Register map (physical, one wave, two waves per SIMD so at most 256 VGPRs):
  v0..v63    O^T accumulators (4 blocks of 32 head columns)
  v64..v127  scores, two sets (tile parity) x two 32-key blocks
  v128..v159 Q^T fragments (B operands of the score MFMAs)
  v160..v175 packed P (B operands of the P.V MFMAs)
  v176..v207 LDS operand ring (8 slots x 4)
  v208..v211 m, l, lh, m * c
  v212..v223 temporaries
SGPR pairs s[80:81] and s[82:83] carry the K and V DMA source addresses.

Run: python gen_fwd_loop.py <output.inc>   (the build runs it before compiling)
"""
import sys

TYPES = {"BF16": ("v_mfma_f32_32x32x16_bf16", "v_cvt_pk_bf16_f32", "v_dot2c_f32_bf16", "0x3f803f80"),
         "F16": ("v_mfma_f32_32x32x16_f16", "v_cvt_pk_f16_f32", "v_dot2c_f32_f16", "0x3c003c00")}
HEAD_DIMS = (128,)   # at d = 64 this schedule (bitwise equal) measured 1-2% faster without a causal mask
                     # and 4.4% slower with one (B1 H32 N8192), so d = 64 keeps the C++ step

AHEAD = 6            # LDS operand reads in flight ahead of their MFMA
RING_SLOTS = 8       # the ring v176..v207
# the read issued after MFMA i fills slot (i + AHEAD) % RING_SLOTS, which must not be
# the slot of MFMA i or of any MFMA still waiting for its operand
assert AHEAD < RING_SLOTS
O0, SB, Q0, P0, R0 = 0, (64, 96), 128, 160, 176
VM, VL, VLH, VMC = 208, 209, 210, 211
MXA, MXB, MX, SWP, TS, ALPHA, MNEW = 212, 213, 214, 215, 216, 217, 218
SUMT = (219, 220, 221, 222, 223)
H1 = 212             # second lh chain (free while the maximum is not being formed)
NREG = 224

# wait states (instructions in between) before a reader of a result
W_VALU_TO_MFMA, W_MFMA_TO_ANY, W_TRANS_TO_VALU, W_DOT_TO_OTHER = 2, 19, 1, 3


def vr(a, n=1):
    return "v%d" % a if n == 1 else "v[%d:%d]" % (a, a + n - 1)


class Stream:
    """Emitted instructions plus the last writer of every VGPR, for the checker."""

    def __init__(self):
        self.out = []
        self.pos = 0
        self.last = {}  # vgpr -> (position, kind, the writer's destination range)

    def raw(self, text, slots=0):
        self.out.append(text)
        self.pos += slots

    def nop(self, n):
        while n > 0:
            k = min(n, 8)
            self.out.append("s_nop %d" % (k - 1))
            self.pos += k
            n -= k

    def _wait(self, regs, kind, acc):
        need = 0
        for r in regs:
            if r not in self.last:
                continue
            p, wk, rng = self.last[r]
            between = self.pos - p - 1
            if wk == "mfma":
                if kind == "mfma" and acc == rng:
                    continue  # accumulation into the same registers
                need = max(need, W_MFMA_TO_ANY - between)
            elif wk == "dot":
                if kind == "dot" and acc == rng:
                    continue
                need = max(need, W_DOT_TO_OTHER - between)
            elif wk in ("valu", "trans") and kind == "mfma":
                need = max(need, W_VALU_TO_MFMA - between)
            elif wk == "trans" and kind in ("valu", "trans", "dot"):
                need = max(need, W_TRANS_TO_VALU - between)
        self.nop(need)

    def ins(self, text, kind, reads=(), writes=(), acc=None):
        """kind: valu, trans, dot, mfma, ds (LDS read: waited by lgkmcnt), salu."""
        if kind not in ("salu", "ds"):
            self._wait(list(reads), kind, acc)
            if kind != "mfma":
                self._wait(list(writes), kind, acc)
        self.out.append(text)
        rng = tuple(writes) if kind in ("mfma", "dot") else None
        for r in writes:
            self.last[r] = (self.pos, kind, rng)
        self.pos += 1


def generate(T, D):
    mfma, cvt, dot2, ones = TYPES[T]
    KS, DB, CG = D // 16, D // 32, D // 32
    TBB = 64 * D * 2                  # bytes of one 64-row tile
    NM = 2 * KS + 4 * DB              # MFMAs per step
    PER_WAVE = (64 // 16) * CG // 4   # DMA instructions per wave and tile
    S = Stream()
    labels = [0]

    def label(name):
        labels[0] += 1
        return "L_%s_%d_%%=" % (name, labels[0])

    def frag_blk(rb, ks):      # byte offset of a 128-bit row-fragment block in a tile
        return (2 * rb * CG + ks // 2) * 1024

    def tr_blk(rs, db):        # byte offset of a transpose-read block in a tile
        return (rs * CG + db) * 1024

    def mfmas(p):
        """The step's MFMAs in order: scores of the next tile (K buffer 1-p), then P.V (V buffer p)."""
        out = []
        for ks in range(KS):
            for kb in range(2):
                out.append(dict(reads=[("ds_read_b128", "%%[k%d]" % (ks & 1), (1 - p) * TBB + frag_blk(kb, ks), 4)],
                                dst=SB[1 - p] + 16 * kb, b=Q0 + 4 * ks, first=ks == 0, pv=None))
        for kb in range(2):
            for t in range(2):
                for db in range(DB):
                    off = 2 * TBB + p * TBB + tr_blk(2 * kb + t, db)
                    out.append(dict(reads=[("ds_read_b64_tr_b16", "%[v0]", off, 2), ("ds_read_b64_tr_b16", "%[v1]", off, 2)],
                                    dst=O0 + 16 * db, b=P0 + 8 * kb + 4 * t, first=False, pv=(kb, t)))
        return out

    def exps(p, kb):
        s = SB[p] + 16 * kb
        ops = []
        for e in range(0, 16, 2):
            for x in (s + e, s + e + 1):
                ops.append(("v_fma_f32 %s, %s, %%[c], -%s" % (vr(x), vr(x), vr(VMC)), "valu", [x, VMC], [x]))
            for x in (s + e, s + e + 1):
                ops.append(("v_exp_f32 %s, %s" % (vr(x), vr(x)), "trans", [x], [x]))
        return ops

    def packs(p, kb):
        s = SB[p] + 16 * kb
        ops = []
        for t in range(2):
            for q in range(4):
                d, a = P0 + 8 * kb + 4 * t + q, s + 8 * t + 2 * q
                ops.append(("%s %s, %s, %s" % (cvt, vr(d), vr(a), vr(a + 1)), "valu", [a, a + 1], [d]))
        return ops

    def sums(p, kb):
        # l += ((p0+p4)+(p8+p12) + (p1+p5)+(p9+p13)) + ((p2+p6)+(p10+p14) + (p3+p7)+(p11+p15))
        s, t = SB[p] + 16 * kb, SUMT
        ops = []

        def add(d, a, b):
            ops.append(("v_add_f32 %s, %s, %s" % (vr(d), vr(a), vr(b)), "valu", [a, b], [d]))
        for i in range(4):
            add(t[i], s + i, s + i + 4)
            add(t[4], s + i + 8, s + i + 12)
            add(t[i], t[i], t[4])
        add(t[0], t[0], t[1])
        add(t[2], t[2], t[3])
        add(t[0], t[0], t[2])
        add(VL, VL, t[0])
        return ops

    def lh_sums(kb):
        # two chains of v_dot2c against (1, 1): lh += both halves of the rounded weights
        ops = [("v_mov_b32 %s, 0" % vr(H1), "valu", [], [H1])]
        for q in range(4):
            a, b = P0 + 8 * kb + q, P0 + 8 * kb + 4 + q
            ops.append(("%s %s, %s, %s" % (dot2, vr(VLH), ones, vr(a)), "dot", [a, VLH], [VLH]))
            ops.append(("%s %s, %s, %s" % (dot2, vr(H1), ones, vr(b)), "dot", [b, H1], [H1]))
        ops.append(("v_add_f32 %s, %s, %s" % (vr(VLH), vr(VLH), vr(H1)), "valu", [VLH, H1], [VLH]))
        return ops

    def maximum(q, grow, back):
        """Row maximum of score set q (both halves of the wave), the lazy-rescale
        test, and a branch to the out-of-line grow block when any row grows."""
        s = SB[q]
        ops = []
        for acc, el in ((MXA, list(range(s, s + 16))), (MXB, list(range(s + 16, s + 32)))):
            ops.append(("v_max3_f32 %s, %s, %s, %s" % (vr(acc), vr(el[0]), vr(el[1]), vr(el[2])), "valu", el[:3], [acc]))
            for i in range(3, 15, 2):
                ops.append(("v_max3_f32 %s, %s, %s, %s" % (vr(acc), vr(acc), vr(el[i]), vr(el[i + 1])), "valu",
                            [acc, el[i], el[i + 1]], [acc]))
            ops.append(("v_max_f32 %s, %s, %s" % (vr(acc), vr(acc), vr(el[15])), "valu", [acc, el[15]], [acc]))
        ops += [("v_max_f32 %s, %s, %s" % (vr(MX), vr(MXA), vr(MXB)), "valu", [MXA, MXB], [MX]),
                ("v_mov_b32 %s, %s" % (vr(SWP), vr(MX)), "valu", [MX], [SWP]),
                ("", "nop2", [], []),
                ("v_permlane32_swap_b32 %s, %s" % (vr(MX), vr(SWP)), "valu", [MX, SWP], [MX, SWP]),
                ("", "nop2", [], []),
                ("v_max_f32 %s, %s, %s" % (vr(MX), vr(MX), vr(SWP)), "valu", [MX, SWP], [MX]),
                # grow = mx > m && !(8 >= (mx - m) c): with m = -inf the product is +inf, or NaN when c = 0
                ("v_sub_f32 %s, %s, %s" % (vr(TS), vr(MX), vr(VM)), "valu", [MX, VM], [TS]),
                ("v_mul_f32 %s, %%[c], %s" % (vr(TS), vr(TS)), "valu", [TS], [TS]),
                ("v_cmp_nge_f32_e32 vcc, 0x41000000, %s" % vr(TS), "valu", [TS], []),
                ("v_cmp_gt_f32_e64 %%[g], %s, %s" % (vr(MX), vr(VM)), "valu", [MX, VM], []),
                ("s_and_b64 %[f], vcc, %[g]", "salu", [], []),
                ("s_cbranch_scc1 %s" % grow, "salu", [], []),
                ("%s:" % back, "label", [], [])]
        return ops

    def emit(ops):
        for (t, k, r, w) in ops:
            if k == "nop2":
                S.nop(2)
            elif k == "label":
                S.raw(t)
            elif k == "salu":
                S.ins(t, "salu")
            else:
                S.ins(t, k, r, w, acc=tuple(w) if k == "dot" else None)

    def grow_block(grow, back):
        # any row grew: all rows take m' = max(m, mx), alpha = (m == -inf) ? 0 : 2^((m - m') c), mc = m' c
        S.raw("%s:" % grow)
        S.nop(2)
        for t in ("v_max_f32 %s, %s, %s" % (vr(MNEW), vr(VM), vr(MX)),
                  "v_sub_f32 %s, %s, %s" % (vr(TS), vr(VM), vr(MNEW)),
                  "v_mul_f32 %s, %%[c], %s" % (vr(TS), vr(TS)),
                  "v_exp_f32 %s, %s" % (vr(ALPHA), vr(TS)),
                  "v_cmp_neq_f32_e64 %%[g], %%[ninf], %s" % vr(VM),
                  "s_nop 1",
                  "v_cndmask_b32_e64 %s, 0, %s, %%[g]" % (vr(ALPHA), vr(ALPHA)),
                  "v_mov_b32 %s, %s" % (vr(VM), vr(MNEW)),
                  "s_nop 1",
                  "v_mul_f32 %s, %%[c], %s" % (vr(VMC), vr(VM)),
                  "v_cmp_neq_f32_e64 %%[g], %%[ninf], %s" % vr(VM),
                  "s_nop 1",
                  "v_cndmask_b32_e64 %s, 0, %s, %%[g]" % (vr(VMC), vr(VMC)),
                  "s_nop 1",
                  "s_branch %s" % back):
            S.raw(t)

    def rescale(nops=True):
        if nops:
            S.nop(24)
        for i in range(16 * DB):
            S.raw("v_mul_f32 %s, %s, %s" % (vr(O0 + i), vr(ALPHA), vr(O0 + i)))
        S.raw("v_mul_f32 %s, %s, %s" % (vr(VL), vr(VL), vr(ALPHA)))
        S.raw("v_mul_f32 %s, %s, %s" % (vr(VLH), vr(VLH), vr(ALPHA)))

    def dma(p, i):
        """i < PER_WAVE: a block of K(j+2) into K buffer p; else a block of V(j+1) into V buffer 1-p."""
        kv = i >= PER_WAVE
        i %= PER_WAVE
        m0 = "%%[mv%d]" % (1 - p) if kv else "%%[mk%d]" % p
        S.raw("s_add_u32 m0, %s, %d" % (m0, 4096 * i), 1)
        S.nop(1)
        S.raw("global_load_lds_dwordx4 %%[g%d], %s" % (i, "s[82:83]" if kv else "s[80:81]"), 1)

    def step(p):
        """Key tile j of parity p: its scores are in set p; the next tile's go to set 1-p."""
        resc, resc_back = label("rescale"), label("rescale_back")
        grow, grow_back = label("grow"), label("grow_back")
        # every wave's DMA of K(j+1), V(j) has landed; every wave is done with K(j), V(j-1)
        S.raw("s_waitcnt vmcnt(0)", 1)
        S.raw("s_barrier", 1)
        S.raw("s_cmp_lg_u64 %[f], 0", 1)
        S.raw("s_cbranch_scc1 %s" % resc, 1)
        S.raw("%s:" % resc_back)
        for i in range(2 * PER_WAVE):
            dma(p, i)
        L = mfmas(p)

        def reads(i):
            if i < NM:
                slot = R0 + 4 * (i % RING_SLOTS)
                for k, (op, addr, off, n) in enumerate(L[i]["reads"]):
                    dst = slot + (2 * k if n == 2 else 0)
                    S.ins("%s %s, %s offset:%d" % (op, vr(dst, n), addr, off), "ds", [], list(range(dst, dst + n)))
        for i in range(min(AHEAD, NM)):
            reads(i)
        S.raw("s_setprio 1")
        ops = exps(p, 0) + packs(p, 0) + exps(p, 1) + packs(p, 1)
        ops += sums(p, 0) + lh_sums(0) + sums(p, 1) + lh_sums(1) + maximum(1 - p, grow, grow_back)
        counted = ("valu", "trans", "dot")
        total = sum(1 for o in ops if o[1] in counted)
        pack_end = (len(exps(p, 0)) + len(packs(p, 0)), 2 * (len(exps(p, 0)) + len(packs(p, 0))))
        done, oi = 0, 0

        def take():
            nonlocal done, oi
            t, k, r, w = ops[oi]
            oi += 1
            done += k in counted
            emit([(t, k, r, w)])
        for i, M in enumerate(L):
            later = sum(len(L[k]["reads"]) for k in range(i + 1, min(i + AHEAD, NM)))
            S.raw("s_waitcnt lgkmcnt(%d)" % min(later, 15), 1)
            slot = R0 + 4 * (i % RING_SLOTS)
            dst = list(range(M["dst"], M["dst"] + 16))
            rd = list(range(slot, slot + 4)) + list(range(M["b"], M["b"] + 4)) + ([] if M["first"] else dst)
            S.ins("%s %s, %s, %s, %s" % (mfma, vr(M["dst"], 16), vr(slot, 4), vr(M["b"], 4),
                                         "0" if M["first"] else vr(M["dst"], 16)), "mfma", rd, dst, acc=tuple(dst))
            reads(i + AHEAD)
            # the packed P of key block kb must exist before its first P.V MFMA
            if i + 1 < NM and L[i + 1]["pv"] is not None and L[i + 1]["pv"][1] == 0:
                while oi < pack_end[L[i + 1]["pv"][0]]:
                    take()
            while done < round((i + 1) * total / NM) and oi < len(ops):
                take()
        while oi < len(ops):
            take()
        S.raw("s_setprio 0")
        # the DMA sources advance by one tile
        S.raw("s_add_u32 s80, s80, %d" % TBB)
        S.raw("s_addc_u32 s81, s81, 0")
        S.raw("s_add_u32 s82, s82, %d" % TBB)
        S.raw("s_addc_u32 s83, s83, 0", 4)
        return resc, resc_back, grow, grow_back

    # entry: the scores of the first tile come from MFMAs the compiler issued
    S.nop(24)
    S.raw("v_mul_f32 %s, %%[c], %s" % (vr(VMC), vr(VM)))
    S.raw("v_cmp_neq_f32_e64 %%[g], %%[ninf], %s" % vr(VM))
    S.raw("s_nop 1")
    S.raw("v_cndmask_b32_e64 %s, 0, %s, %%[g]" % (vr(VMC), vr(VMC)))
    S.raw("s_cmp_eq_u32 %[par], 0")
    S.raw("s_cbranch_scc0 L_entry1_%=")
    out_of_line = []
    for par in (0, 1):
        S.raw("L_entry%d_%%=:" % par)
        g, b = label("grow"), label("grow_back")
        emit(maximum(par, g, b))
        out_of_line.append((None, None, g, b))
        S.raw("s_branch L_step%d_%%=" % par)
    S.last = {}
    for par in (0, 1):
        S.raw("L_step%d_%%=:" % par)
        out_of_line.append(step(par))
        S.raw("s_sub_u32 %[n], %[n], 1")
        S.raw("s_cmp_eq_u32 %[n], 0")
        S.raw("s_cbranch_scc1 L_exit_%=", 3)
    S.raw("s_branch L_step0_%=")
    for (resc, resc_back, grow, grow_back) in out_of_line:
        if resc:
            S.raw("%s:" % resc)
            rescale()
            S.nop(2)
            S.raw("s_branch %s" % resc_back)
        grow_block(grow, grow_back)
    # exit: this wave's DMA has landed; a rescale decided in the last step is applied here
    S.raw("L_exit_%=:")
    S.raw("s_waitcnt vmcnt(0)")
    S.raw("s_cmp_lg_u64 %[f], 0")
    S.raw("s_cbranch_scc0 L_done_%=")
    rescale()
    S.raw("L_done_%=:")
    S.nop(24)  # the compiler's code after the statement may read MFMA results at once
    return S.out


def function(T, D):
    KS, DB = D // 16, D // 32
    PER_WAVE = (64 // 16) * (D // 32) // 4
    body = "\\n\\t".join(generate(T, D))
    outs = ['"+{v[%d:%d]}"(o[%d])' % (O0 + 16 * db, O0 + 16 * db + 15, db) for db in range(DB)]
    outs += ['"+{v[%d:%d]}"(s%d[%d])' % (SB[p] + 16 * kb, SB[p] + 16 * kb + 15, p, kb) for p in range(2) for kb in range(2)]
    outs += ['"+{v%d}"(m)' % VM, '"+{v%d}"(l)' % VL, '"+{v%d}"(lh)' % VLH, '[n] "+s"(n)', '"+{s[80:81]}"(kbase)',
             '"+{s[82:83]}"(vbase)', '[f] "=&s"(f)', '[g] "=&s"(g2)']
    ins = ['"{v[%d:%d]}"(q[%d])' % (Q0 + 4 * ks, Q0 + 4 * ks + 3, ks) for ks in range(KS)]
    ins += ['[k0] "v"(k0)', '[k1] "v"(k1)', '[v0] "v"(v0)', '[v1] "v"(v1)']
    ins += ['[g%d] "v"(g[%d])' % (i, i) for i in range(PER_WAVE)]
    ins += ['[c] "s"(c)', '[ninf] "s"(ninf)', '[par] "s"(par)', '[mk0] "s"(mk0)', '[mk1] "s"(mk1)',
            '[mv0] "s"(mv0)', '[mv1] "s"(mv1)']
    clobbers = ", ".join('"v%d"' % r for r in range(P0, NREG) if r not in (VM, VL, VLH))
    return "\n".join([
        "template <>",
        "__device__ inline void fwd_unmasked_run<%s, %d>(%s) {" % (T, D, SIGNATURE % {"DB": DB, "KS": KS}),
        "    uint64_t f, g2;",
        "    const uint32_t ninf = 0xff800000u;",
        '    asm volatile("%s"' % body,
        "                 : " + ",\n                   ".join(outs),
        "                 : " + ",\n                   ".join(ins),
        '                 : %s, "vcc", "scc", "m0", "memory");' % clobbers,
        "}"])


SIGNATURE = ("f32x16 (&o)[%(DB)s], f32x16 (&s0)[2], f32x16 (&s1)[2], float& m, float& l, float& lh, "
             "const u32x4 (&q)[%(KS)s], uint32_t k0, uint32_t k1, uint32_t v0, uint32_t v1, const uint32_t (&g)[4], "
             "float c, uint32_t par, uint32_t mk0, uint32_t mk1, uint32_t mv0, uint32_t mv1, uint64_t kbase, "
             "uint64_t vbase, uint32_t n")

HEADER = """// attn_fwd_loop.inc -- generated by gen_fwd_loop.py (run by the build); do not edit.
//
// fwd_unmasked_run<T, D>: n consecutive unmasked key tiles of the forward
// kernel's loop, starting at a tile of parity par, as one inline-assembly
// statement.  On entry the scores of the first tile are in s<par>, K of the
// next tile and V of the first are in LDS, and the DMA sources kbase / vbase
// point at K two tiles and V one tile ahead (plus this wave's block offset);
// on exit the state is the one the C++ step expects for the tile after the
// last: scores in s<par of that tile>, m / l / lh / o updated, DMA landed.
// Inputs: k0 / k1 / v0 / v1 LDS read addresses (buffer 0), g the DMA lane
// offsets of the wave's blocks, mk / mv the DMA LDS destinations of the two
// K and V buffers for this wave, c = scale * log2(e) (non-negative).
// n >= 1: the statement counts tiles down to zero, so a count of 0 would not end.
"""


def main(path):
    parts = [HEADER,
             "template <class T, int D>",
             "__device__ inline void fwd_unmasked_run(%s);" % (SIGNATURE % {"DB": "D / 32", "KS": "D / 16"})]
    for T in ("BF16", "F16"):
        for D in HEAD_DIMS:
            parts.append(function(T, D))
    text = "\n".join(parts[:3]) + "\n\n" + "\n\n".join(parts[3:]) + "\n"
    old = open(path).read() if __import__("os").path.exists(path) else None
    if old != text:
        with open(path, "w") as fh:
            fh.write(text)


if __name__ == "__main__":
    main(sys.argv[1])
