"""Properties of the library's gfx950 device code that no GPU test shows
directly, checked on the assembly compiled here (device code only, the
library's own device flags; no GPU needed):

- every 16-byte store of the kernels is the hand-written one
  (global_store_dwordx4 ... sc1 nt): non-temporal at device scope;
- each of those stores is followed at once by s_nop.  The store is an
  inline-asm statement the compiler does not see, and on gfx9 a VALU write
  to the data registers of a store of more than 8 bytes needs one wait state
  after it; without it the d = 8 fused kernel overwrote part of q's result
  before the store had read it;
- no kernel uses private (scratch) memory;
- no packed fp32 instruction appears (the library is built without them).
"""
import os
import re
import subprocess

import pytest

from sequence_attention_relayout_amd import build as B

KERNELS = os.path.join(B.CSRC, "kernels.hip")


def compile_asm(tmp_path):
    out = os.path.join(tmp_path, "kernels.s")
    flags = [f for f in B.DEVICE_FLAGS if f != "-fPIC"]
    subprocess.run([os.path.join(B.ROCM, "bin", "hipcc"), *flags, "--cuda-device-only", "-S",
                    f"-I{B.CSRC}", KERNELS, "-o", out], check=True, capture_output=True)
    with open(out) as f:
        return f.read()


def instructions(text):
    """(function, instruction) pairs in order: labels, directives and
    comments dropped."""
    fn, out = None, []
    for raw in text.splitlines():
        line = raw.strip()
        m = re.match(r"^([A-Za-z_][\w.$]*):", line)
        if m:
            if not m.group(1).startswith("."):
                fn = m.group(1)
            continue
        if not line or line.startswith((";", ".", "//")):
            continue
        out.append((fn, line))
    return out


def store_problems(text):
    """Every 16-byte store that lacks the sc1 nt policy or is not followed at
    once by s_nop, as (function, store, next instruction)."""
    ins = instructions(text)
    bad = []
    for i, (fn, line) in enumerate(ins):
        if not line.startswith("global_store_dwordx4"):
            continue
        nxt = ins[i + 1][1] if i + 1 < len(ins) else ""
        if not re.search(r"\bsc1\b", line) or not re.search(r"\bnt\b", line) \
                or not nxt.startswith("s_nop"):
            bad.append((fn, line, nxt))
    return bad


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    return compile_asm(str(tmp_path_factory.mktemp("asm")))


def test_checker_catches_a_store_without_its_wait_state():
    good = "k:\n\tglobal_store_dwordx4 v[0:1], v[2:5], off sc1 nt\n\ts_nop 0\n\t;;#ASMEND\n\ts_endpgm\n"
    bad = "k:\n\tglobal_store_dwordx4 v[0:1], v[2:5], off sc1 nt\n\tv_mul_f32_e32 v2, v3, v4\n"
    plain = "k:\n\tglobal_store_dwordx4 v[0:1], v[2:5], off nt\n\ts_nop 0\n"
    assert store_problems(good) == []
    assert len(store_problems(bad)) == 1
    assert len(store_problems(plain)) == 1


def test_every_store_is_device_scope_and_followed_by_its_wait_state(asm):
    stores = [l for _, l in instructions(asm) if l.startswith("global_store_dwordx4")]
    # relayout (4 instantiations), plane copy, fused (14 instantiations, 2 stores each)
    assert len(stores) >= 4 + 1 + 14 * 2
    assert store_problems(asm) == []
    # no narrower or flat store slips in beside them
    assert not [l for _, l in instructions(asm)
                if re.match(r"(global|flat|buffer)_store", l) and "dwordx4" not in l]


def test_no_kernel_uses_private_memory(asm):
    sizes = re.findall(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", asm)
    assert len(sizes) >= 19
    assert set(sizes) == {"0"}


def test_no_packed_fp32_instructions(asm):
    assert not re.search(r"\bv_pk_(add|mul|fma)_f32\b", asm)
