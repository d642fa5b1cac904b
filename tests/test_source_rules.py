"""Source-level checks of the HIP sources that need no GPU.

* A wave-uniform 64-bit address rebuilt from two __builtin_amdgcn_readfirstlane
  halves must widen each half through uint32_t: the builtin returns a signed
  int, and a low word with bit 31 set would otherwise sign-extend into the
  high word (a DMA source address with its upper half all ones).
* The committed attn_fwd_loop.inc, attn_dq_loop.inc and attn_dkdv_loop.inc are
  what their generators write.
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
