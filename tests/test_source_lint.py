"""Source checks that need no GPU.

clang's __builtin_bit_cast applied to an element of an ext_vector_type value
(`__builtin_bit_cast(float, v[1])`) reads element 0 of the vector instead of
the named element. The kernels copy such elements into a scalar first; this
keeps the pattern out of every HIP source."""
import glob
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "mla_attention_under_amd", "csrc")
PATTERN = re.compile(r"__builtin_bit_cast\(\s*[\w:<> ]+\s*,\s*[\w.]+\s*\[")


def test_no_bit_cast_of_subscripted_elements():
    hits = []
    for path in sorted(glob.glob(os.path.join(CSRC, "*"))):
        for n, line in enumerate(open(path), 1):
            if PATTERN.search(line):
                hits.append(f"{os.path.basename(path)}:{n}: {line.strip()}")
    assert not hits, "\n".join(hits)


def test_pattern_catches_the_bad_form():
    assert PATTERN.search("x = __builtin_bit_cast(float, sw[1]);")
    assert PATTERN.search("f(__builtin_bit_cast(bf16x2_t, w[e]), one)")
    assert not PATTERN.search("__builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1))")
    assert not PATTERN.search("__builtin_bit_cast(bf16x2_t, pp)")
