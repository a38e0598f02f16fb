"""The oracle's pins must catch plausible mistakes.

Each case copies the oracle's C source, plants one mistake by a textual edit
(a wrong padding sign, swapped filter indices, a dropped stride, a dropped
tap, an off-by-one extent, a flipped kernel), compiles it on the CPU, and
checks that the pin set of ``test_oracle_pins`` rejects it. The planted copies
live in a temporary directory; the oracle itself is untouched.
"""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

MUTANTS = {
    "pad_sign_rows": ("int64_t ih = ho * s + kh - p;", "int64_t ih = ho * s + kh + p;"),
    "swapped_filter_taps": ("wc[kh * KW + kw]", "wc[kw * KH + kh]"),
    "dropped_stride": ("int64_t iw = wo * s + kw - p;", "int64_t iw = wo + kw - p;"),
    "dropped_last_tap": ("for (int64_t kw = 0; kw < KW; ++kw) {", "for (int64_t kw = 0; kw + 1 < KW; ++kw) {"),
    "extent_off_by_one": ("return span / s + 1;", "return (span + s - 1) / s + 1;"),
    "flipped_kernel": ("wc[kh * KW + kw]", "wc[(KH - 1 - kh) * KW + (KW - 1 - kw)]"),
}


def _pins_pass(orc) -> bool:
    """A compact form of the pin set: library conv on several shapes, and
    the Table I extent of cv4 (the one with a non-divisible span)."""
    if orc.out_extent(224, 7, 2, 0) != 109 or orc.out_extent(227, 11, 4, 0) != 55:
        return False
    rng = np.random.default_rng(0)
    for (N, C, H, W, Co, KH, KW, s, p) in [(1, 2, 7, 8, 3, 3, 2, 1, 1), (2, 3, 9, 9, 2, 3, 3, 2, 1),
                                           (1, 1, 6, 7, 2, 2, 3, 1, 0), (1, 2, 11, 10, 2, 5, 4, 3, 2)]:
        x = rng.standard_normal((N, C, H, W))
        w = rng.standard_normal((Co, C, KH, KW))
        try:
            y = orc.conv2d(x, w, s, p)
        except ValueError:
            return False
        ref = F.conv2d(torch.from_numpy(x), torch.from_numpy(w), stride=s, padding=p).numpy()
        if y.shape != ref.shape or not np.allclose(y, ref, rtol=1e-12, atol=1e-12):
            return False
    return True


def test_unmodified_oracle_passes(orc):
    assert _pins_pass(orc)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, name
    mutated = tmp_path / f"mutant_{name}.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.build(str(mutated), str(tmp_path / f"libmutant_{name}.so"))
    assert not _pins_pass(oracle.Oracle(lib)), f"pins did not catch mutant {name}"
