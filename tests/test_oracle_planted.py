"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (never in the
committed file), builds it on the CPU, and runs the pins of
test_oracle_pins.py against it: at least one pin must fail.  This shows that the
pins constrain every step (rounding, scale, division, nibble order, scale
indexing, group range, accumulation order-independent parts).
"""
import numpy as np
import pytest

from oracle import oracle
import tests.test_oracle_pins as pins

PINS = [
    lambda o: pins.test_quantize_hand_cases(o),
    lambda o: pins.test_pack_bytes_fixture(o),
    lambda o: pins.test_quantize_invariants(o, "outlier", 128),
    lambda o: pins.test_gemm_unit_scales_is_integer_matmul(o, 128),
    lambda o: pins.test_gemm_per_channel_closed_form(o),
    lambda o: pins.test_gemm_fp64_bruteforce_bound(o, 128, 128),
    lambda o: pins.test_gemm_fp64_bruteforce_bound(o, 128, 1024),
    lambda o: pins.test_gemm_fp64_bruteforce_bound(o, 32, 32),
]

# (name, text in the oracle source, replacement)
MUTANTS = [
    ("round half away from zero", "float v = nearbyintf(", "float v = roundf("),
    ("multiply by reciprocal", "oracle_f16_to_f32(xr[k]) / sc", "oracle_f16_to_f32(xr[k]) * (1.0f / sc)"),
    ("scale absmax/8", "amax / 7.0f", "amax / 8.0f"),
    # (raising the clamp to 8 would be an equivalent mutant: |x/s| never rounds past 7)
    ("clamp too tight", "if (v > 7.0f) v = 7.0f;", "if (v > 6.0f) v = 6.0f;"),
    ("odd k in low nibble", "if (k % 2 == 0)\n                    qr[k / 2] |= nibble_of(code);",
     "if (k % 2 == 1)\n                    qr[k / 2] |= nibble_of(code);"),
    ("unsigned nibbles", "return nib >= 8 ? (int)nib - 16 : (int)nib;", "return (int)nib;"),
    ("weight scale indexed by activation group size", "s_w[n * Gw + (j * gs) / gw]",
     "s_w[n * Gw + (j * gs) / ga]"),
    ("last group dropped", "for (int64_t j = 0; j < G; ++j) {\n                /* exact",
     "for (int64_t j = 0; j + 1 < G; ++j) {\n                /* exact"),
    ("group range off by one", "for (int64_t k = j * gs; k < (j + 1) * gs; ++k)\n                    pj +=",
     "for (int64_t k = j * gs + 1; k < (j + 1) * gs; ++k)\n                    pj +="),
    ("sign of the accumulate", "acc = acc + t;", "acc = acc - t;"),
    ("weight row taken from the activation", "(int64_t)cw[n * K + k]", "(int64_t)ca[(n % M) * K + k]"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = oracle.source()
    assert src.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    mut = oracle.build_variant(src.replace(old, new), str(tmp_path / "mutant.so"))
    failures = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mut)
        except (AssertionError, oracle.OracleError, ValueError):
            failures += 1
    assert failures >= 1, f"no pin caught the planted mistake: {name}"
