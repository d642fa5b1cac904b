"""Source-level checks of the HIP sources that need no GPU.

* A wave-uniform 64-bit address rebuilt from two __builtin_amdgcn_readfirstlane
  halves must widen each half through uint32_t: the builtin returns a signed
  int, and a low word with bit 31 set would otherwise sign-extend into the
  high word (a DMA source address with its upper half all ones).
* The committed attn_fwd_loop.inc, attn_dq_loop.inc and attn_dkdv_loop.inc are
  what their generators write.
* In each generated loop, no path has more than 15 LDS instructions in flight
  (lgkmcnt is a 4-bit counter), and every statement ends with none in flight.
* No packed-fp32 vector instruction appears in the generated loops or the HIP
  sources: the build compiles with packed fp32 disabled, and hand-written code
  must not bring it back.
"""
import os
import re
import sys

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "io_aware_exact_06_amd", "csrc")


def sources():
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h", ".cpp", ".inc")):
            with open(os.path.join(CSRC, name)) as fh:
                yield name, fh.read()


def test_readfirstlane_widened_through_uint32():
    bad = []
    for name, text in sources():
        for m in re.finditer(r"\(\s*u?int64_t\s*\)\s*__builtin_amdgcn_readfirstlane", text):
            bad.append("%s:%d" % (name, text.count("\n", 0, m.start()) + 1))
    assert not bad, "readfirstlane widened to 64 bits without a uint32_t cast: %s" % bad


def test_generated_loops_in_sync(tmp_path):
    sys.path.insert(0, CSRC)
    try:
        import gen_dkdv_loop
        import gen_dq_loop
        import gen_fwd_loop
    finally:
        sys.path.pop(0)
    for gen, name in ((gen_fwd_loop, "attn_fwd_loop.inc"), (gen_dkdv_loop, "attn_dkdv_loop.inc"),
                      (gen_dq_loop, "attn_dq_loop.inc")):
        out = tmp_path / name
        gen.main(str(out))
        with open(os.path.join(CSRC, name)) as fh:
            assert fh.read() == out.read_text(), name


def lds_in_flight(lines):
    """Upper bound of the LDS instructions in flight before each line of a
    generated statement, over every path through its labels and branches:
    ds_* adds one (saturating at 16), s_waitcnt lgkmcnt(k) caps the count at k, a label takes the
    maximum over its fall-through and every branch to it (iterated to a fixed
    point, so that backward branches count).  Returns (maximum, count at end)."""
    at_label = {}
    for _ in range(len(lines) + 1):
        changed = False
        n, live, mx = 0, True, 0
        for line in lines:
            op = line.split()[0] if line.split() else ""
            if line.endswith(":"):
                lab = line[:-1]
                n = max(n if live else 0, at_label.get(lab, 0))
                live = True
                continue
            if not live:
                continue
            if op.startswith("ds_"):
                n = min(n + 1, 16)  # 16: already over the counter's range
                mx = max(mx, n)
            m = re.match(r"s_waitcnt\s.*lgkmcnt\((\d+)\)", line)
            if m:
                n = min(n, int(m.group(1)))
            if op.startswith(("s_branch", "s_cbranch")):
                target = line.split()[1]
                if n > at_label.get(target, -1):
                    at_label[target] = n
                    changed = True
                if op == "s_branch":
                    live = False
        if not changed:
            return mx, n
    raise AssertionError("no fixed point")


def test_generated_loops_lds_counter():
    sys.path.insert(0, CSRC)
    try:
        import gen_dkdv_loop
        import gen_dq_loop
        import gen_fwd_loop
    finally:
        sys.path.pop(0)
    for gen in (gen_fwd_loop, gen_dq_loop, gen_dkdv_loop):
        for T in ("BF16", "F16"):
            for D in gen.HEAD_DIMS:
                mx, end = lds_in_flight(gen.generate(T, D))
                assert mx <= 15, (gen.__name__, T, D, mx)
                assert end == 0, (gen.__name__, T, D, end)


def test_no_packed_fp32_instructions():
    ops = ["v_pk_" + op + "_f32" for op in ("add", "mul", "fma")]
    bad = []
    for name, text in sources():
        for op in ops:
            if op in text:
                bad.append((name, op))
    sys.path.insert(0, CSRC)
    try:
        import gen_dkdv_loop
        import gen_dq_loop
        import gen_fwd_loop
    finally:
        sys.path.pop(0)
    for gen in (gen_fwd_loop, gen_dq_loop, gen_dkdv_loop):
        for T in ("BF16", "F16"):
            for D in gen.HEAD_DIMS:
                for line in gen.generate(T, D):
                    if any(line.startswith(op) for op in ops):
                        bad.append((gen.__name__, line))
    assert not bad, bad
