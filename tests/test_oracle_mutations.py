"""Planted slips in the CPU oracle must fail at least one pin (CPU only).

Each mutation below is a plausible mistake in `oracle/oracle.c` (a dropped
term, a wrong index, an off-by-one).  The test compiles a mutated copy into a
temporary directory, swaps it in, runs the pins of `test_oracle.py` and checks
that at least one of them fails.  The real oracle is never modified.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = {
    "scale_dropped": ("s[jj] = scale * dot;", "s[jj] = dot;"),
    "no_max_subtraction": ("s[jj] = exp(s[jj] - m);", "s[jj] = exp(s[jj]);"),
    "key_ignores_image_offset": ("k + (j0 + jj) * rs", "k + (jj) * rs"),
    "value_ignores_head": ("v[(j0 + jj) * rs + (int64_t)h * D + d]", "v[(j0 + jj) * rs + d]"),
    "no_normalisation": ("oi[d] = acc / l;", "oi[d] = acc;"),
    "max_from_first_key_only": ("if (s[jj] > m) m = s[jj];", "if (jj == 0) m = s[jj];"),
    "owner_off_by_one": ("t >= cu[b] && t < cu[b + 1]", "t >= cu[b] && t <= cu[b + 1]"),
    "cu_inclusive": ("cu[b + 1] = running;", "cu[b + 1] = running - cnt + (cnt > 0);"),
    "pack_skips_increment": ("                r += 1;\n            }\n        }\n    return r;",
                             "                r += (n > 0);\n            }\n        }\n    return r;"),
    "unpack_no_zero_fill": ("else memset(dst + t * row_bytes, 0, (size_t)row_bytes);", ""),
    "cls_from_last_row": ("if (cls && n == 0)", "if (cls && n == N - 1)"),
    "repack_ignores_keep2": ("            if (keep2[t] != 0) {", "            if (1) {"),
    "repack_cu_not_cumulative": ("        cu2[b + 1] = (int32_t)r;",
                                 "        cu2[b + 1] = (int32_t)(r - (b > 0 ? cu2[b] : 0));"),
}

PINS = [
    (pins.test_scan_pack_hand_fixture, {}),
    (pins.test_pack_unpack_identities, {"seed": 0}),
    (pins.test_pack_unpack_identities, {"seed": 3}),
    (pins.test_scan_all_empty_and_all_kept, {}),
    (pins.test_attention_hand_fixture, {}),
    (pins.test_two_token_logistic_closed_form, {}),
    (pins.test_length_one_returns_v_row_exactly, {}),
    (pins.test_uniform_weights_give_mean_of_v, {"zero": "q"}),
    (pins.test_constant_v_is_returned, {}),
    (pins.test_dominant_logit_is_one_hot_and_finite, {}),
    (pins.test_matches_library_sdpa_per_image, dict(seed=11, B=3, N=9, H=2, D=64)),
    (pins.test_matches_brute_force_padded_masked, {"seed": 1}),
    (pins.test_repack_hand_fixture, {}),
    (pins.test_repack_composes_with_pack, {"seed": 0}),
]


def _fails(fn, kw) -> bool:
    try:
        fn(**kw)
    except Exception:  # AssertionError, ValueError from a rejected result, ...
        return True
    return False


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_slip(name, tmp_path):
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    src = tmp_path / "oracle_mut.c"
    src.write_text(text.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-w",
                           "-o", str(lib), str(src), "-lm"])
    with oracle.use_library(str(lib)):
        caught = [fn.__name__ for fn, kw in PINS if _fails(fn, kw)]
    assert caught, f"no pin caught the planted slip '{name}'"


def test_unmutated_oracle_passes_every_pin():
    assert not [fn.__name__ for fn, kw in PINS if _fails(fn, kw)]
