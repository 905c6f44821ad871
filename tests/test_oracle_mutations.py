"""The oracle pins must catch plausible mistakes.

Each case plants one mistake in a temporary copy of the C oracle (on the CPU),
builds it, and runs the pin suite against it in a subprocess: the suite must
fail.  The shipped oracle is untouched.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "kvq_oracle.c")

MUTANTS = {
    # rounding: half away from zero instead of half to even
    "round_half_away": ("float y = rintf(ratio);", "float y = roundf(ratio);"),
    # offset added before rounding (the literal reading rejected by the spec)
    "offset_first": ("float y = rintf(ratio);", "float y = rintf(ratio + (float)(-(1 << (bits - 1)))) + (float)(1 << (bits - 1));"),
    # eps guard dropped
    "no_eps": ("if (s < KVO_EPS) s = KVO_EPS;", ""),
    # stored scale one fp16 ulp too large (0.1% above the rounded scale)
    "inflated_stored_scale": ("*scale16 = kvo_f32_to_f16(s);", "*scale16 = kvo_f32_to_f16(s * 1.0009765625f);"),
    # affine codes against the fp32 scale before rounding instead of the stored fp16 scale
    "codes_vs_fp32_scale": [
        ("static const float KVO_EPS = 1e-5f;", "static const float KVO_EPS = 1e-5f;\nstatic float kvo_last_s;"),
        ("*scale16 = kvo_f32_to_f16(s);", "*scale16 = kvo_f32_to_f16(s);\n    kvo_last_s = s;"),
        ("float s = kvo_f16_to_f32(scale16);", "float s = kvo_last_s; (void)scale16;"),
    ],
    # symmetric codes rounded half away from zero instead of half to even
    "sym4_round_half_away": ("float y = rintf(xc[i] / df);", "float y = roundf(xc[i] / df);"),
    # symmetric eps floor dropped (an all-zero block divides by zero)
    "sym4_no_eps": ("if (dd < KVO_EPS) dd = KVO_EPS;", ""),
    # symmetric codes against the fp32 d before rounding instead of the stored fp16 d
    "sym4_codes_vs_fp32_scale": ("float df = kvo_f16_to_f32(d16);", "float df = dd;"),
    # fp16 conversion truncates instead of rounding
    "f16_truncate": ("double n = nearbyint(a / quantum);", "double n = floor(a / quantum);"),
    # symmetric quantizer divides by 8 instead of 7
    "sym4_qmax": ("float dd = amax / 7.0f;", "float dd = amax / 8.0f;"),
    # centering bias added instead of subtracted
    "bias_sign": ("if (bias) v = v - bias[d];", "if (bias) v = v + bias[d];"),
    # dequantization drops the zero point
    "dequant_no_zero": ("return (double)v->u[(int64_t)t * D + d] * s + z;\n    }\n    case KVO_SYM4",
                        "return (double)v->u[(int64_t)t * D + d] * s;\n    }\n    case KVO_SYM4"),
    # softmax scale applied twice
    "scale_twice": ("logit[t] = scale * acc;", "logit[t] = scale * scale * acc;"),
    # SnapKV mean over S instead of the clamped window
    "mean_over_S": ("score[j] /= (double)wc;", "score[j] /= (double)S;"),
    # SnapKV window taken from the front
    "window_front": ("for (int i = S - wc; i < S; ++i) {", "for (int i = 0; i < wc; ++i) {"),
    # tie-break prefers the higher position
    "tie_high": ("return (x->i > y->i) - (x->i < y->i);", "return (x->i < y->i) - (x->i > y->i);"),
    # query-row scores divided by S instead of the row count
    "rows_mean_over_S": ("score[j] /= (double)n_rows;", "score[j] /= (double)S;"),
    # max-pool window one short on each side
    "pool_narrow": ("int r = (kernel - 1) / 2;", "int r = (kernel - 1) / 2 - 1;"),
    # RoPE frequencies without the factor 2 in the exponent
    "rope_theta": ("double theta = pow(base, -2.0 * (double)j / (double)D);",
                   "double theta = pow(base, -(double)j / (double)D);"),
    # RoPE: the first component rotated the wrong way
    "rope_sign": ("x[j] = a * c - b * s;", "x[j] = a * c + b * s;"),
    # keys rotated one position past their slot
    "rope_key_pos": ("kvo_rope_rotate(kr, D, base, t);", "kvo_rope_rotate(kr, D, base, t + 1);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    edits = MUTANTS[name]
    if isinstance(edits, tuple):
        edits = [edits]
    src = open(SRC).read()
    for old, new in edits:
        assert src.count(old) >= 1, f"mutation anchor for {name} not found: {old!r}"
        src = src.replace(old, new)
    mut = tmp_path / "kvq_oracle.c"
    mut.write_text(src)
    lib = str(tmp_path / "libmut.so")
    obuild.build(src=str(mut), out=lib)
    env = dict(os.environ, KVQ_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_pins.py")],
                       env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"


def test_control_unmutated_copy_passes(tmp_path):
    """The same harness with an unmodified copy passes (the mutants fail for their mistake)."""
    lib = str(tmp_path / "libctl.so")
    obuild.build(src=SRC, out=lib)
    env = dict(os.environ, KVQ_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_pins.py")],
                       env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
