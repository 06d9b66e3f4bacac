"""Mutation check of the oracle's pins (CPU).

Every parity claim rests on the oracle, so its pins must be able to fail.
Each case below plants one plausible mistake in a copy of
``oracle/fp8w_oracle.c`` (a dropped term, a wrong sign, bias or index, a
transposed operand, a changed reading), builds it with the oracle's own
flags, and runs the oracle pin suite (``tests/test_oracle_*.py``) against
that build in a subprocess.  The suite must fail on every mutant, and pass on
an unmutated copy built the same way (so that a broken harness cannot pass
this test).  The mistakes are planted in the oracle only, on the CPU.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fp8w_oracle.c")

# (name, text in the source, its replacement, how many times the text occurs,
#  which occurrence to replace)
MUTANTS = [
    # encode
    ("ties_away_from_even", "(a == midpoint && (c & 1))", "(a == midpoint)", 1, 0),
    ("saturate_to_nan", "c = 126; /* saturate", "c = 127; /* saturate", 1, 0),
    ("negative_zero_loses_sign", "uint8_t sign = signbit(q) ? 0x80 : 0x00;",
     "uint8_t sign = (q < 0.0f) ? 0x80 : 0x00;", 1, 0),
    # decode
    ("subnormal_exponent", "mag = ldexp((double)m, -9);", "mag = ldexp((double)m, -10);", 1, 0),
    ("decode_bias", "mag = ldexp(1.0 + m / 8.0, e - 7);", "mag = ldexp(1.0 + m / 8.0, e - 8);", 1, 0),
    # fp32 block quantizer
    ("zero_tile_scale", "const float scale = (amax > 0.0f) ? amax / 448.0f : 1.0f;",
     "const float scale = (amax > 0.0f) ? amax / 448.0f : 2.0f;", 1, 0),
    ("scale_divisor", "const float scale = (amax > 0.0f) ? amax / 448.0f : 1.0f;",
     "const float scale = (amax > 0.0f) ? amax / 447.0f : 1.0f;", 1, 0),
    ("reciprocal_multiply", "float q = bf16_to_float(w[r * k + c]) / scale;",
     "float q = bf16_to_float(w[r * k + c]) * (1.0f / scale);", 1, 0),
    # MX quantizer
    ("mx_exponent_sign", "oracle_e4m3_encode(ldexpf(v[c], -e))", "oracle_e4m3_encode(ldexpf(v[c], e))", 1, 0),
    ("mx_bias", "(uint8_t)(e + 127);", "(uint8_t)(e + 128);", 1, 0),
    ("mx_exponent_clamp", "if (e < -127) e = -127;", "if (e < -126) e = -126;", 1, 0),
    ("mx_chunk_offset", "transient[i] = bf16_to_float(w[row0 * k + i]);",
     "transient[i] = bf16_to_float(w[i]);", 1, 0),
    # bf16 block scales (the floor of reading 19 and the scale rounding)
    ("bf16_scale_floor_2^-126", "if (sb == 0) sb = 1;", "if (sb == 0) sb = 0x0080;", 1, 0),
    ("bf16_scale_no_floor", "if (sb == 0) sb = 1;", "if (sb == 0) sb = 0;", 1, 0),
    ("bf16_scale_unrounded", "oracle_round_bf16((double)(amax / 448.0f))",
     "(uint16_t)(oracle_round_bf16((double)(amax / 448.0f)) + (amax / 448.0f > 1e-30f))", 1, 0),
    # per-row quantizer
    ("row_zero_scale", "const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;",
     "const float scale = amax > 0.0f ? amax / 448.0f : 0.5f;", 1, 0),
    # bf16 rounding of the dequantizers
    ("bf16_ties_up", "else pick = (lo % 2 == 0) ? lo : (uint16_t)(lo + 1);",
     "else pick = (uint16_t)(lo + 1);", 1, 0),
    # exact dequantizers and the GEMV references
    ("dequant_block_transposed", "(double)scales[(r / TILE) * tiles_k + c / TILE];",
     "(double)scales[(c / TILE) * tiles_k + r / TILE];", 2, 0),
    ("gemv_block_scale_transposed", "d *= (double)block_scales[(r / TILE) * tiles_k + c / TILE];",
     "d *= (double)block_scales[(c / TILE) * tiles_k + r / TILE];", 2, 1),
    ("gemv_mx_bias", "d = ldexp(d, (int)e8m0[r * groups + c / MX_GROUP] - 127);",
     "d = ldexp(d, (int)e8m0[r * groups + c / MX_GROUP] - 126);", 2, 1),
    ("gemv_signed_bound", "mag += fabs(xv) * fabs(d);", "mag += xv * d;", 3, 2),
    ("gemv_dropped_last_column", "for (int64_t c = 0; c < k; ++c) {\n        double d = oracle_e4m3_decode",
     "for (int64_t c = 0; c < k - 1; ++c) {\n        double d = oracle_e4m3_decode", 2, 1),
    ("format_scale_mx_bias", "MX_GROUP] - 127);\n    case FMT_BLOCK_BF16:",
     "MX_GROUP] - 126);\n    case FMT_BLOCK_BF16:", 1, 0),
    # W8A8 references
    ("act_scale_divisor", "(float)(amax / (float)E4M3_MAX)", "(float)(amax / 447.0f)", 1, 0),
    ("w8a8_drops_act_scale", "const double xv = oracle_e4m3_decode(xc[i * k + c]) * (double)xs;",
     "const double xv = oracle_e4m3_decode(xc[i * k + c]) * (double)(xs > 0.0f);", 1, 0),
]


def _pin_files():
    me = os.path.abspath(__file__)
    files = sorted(f for f in glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py"))
                   if os.path.abspath(f) != me)
    assert files
    return files


def _mutate(src: str, old: str, new: str, count: int, which: int) -> str:
    assert src.count(old) == count, f"{old!r} occurs {src.count(old)} times, expected {count}"
    at = -1
    for _ in range(which + 1):
        at = src.index(old, at + 1)
    return src[:at] + new + src[at + len(old):]


def _run_pins(lib: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, FP8W_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           *_pin_files()]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def _build_and_run(tmp_path, name: str, text: str):
    import oracle
    d = tmp_path / name
    d.mkdir()
    src = d / "fp8w_oracle.c"
    src.write_text(text)
    lib = str(d / "liboracle.so")
    oracle.compile_source(str(src), lib)
    return _run_pins(lib)


@pytest.mark.slow
def test_every_planted_oracle_mistake_fails_a_pin(tmp_path):
    original = open(SRC).read()
    jobs = {"unmutated": original}
    for name, old, new, count, which in MUTANTS:
        jobs[name] = _mutate(original, old, new, count, which)
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        futs = {name: ex.submit(_build_and_run, tmp_path, name, text) for name, text in jobs.items()}
        results = {name: f.result() for name, f in futs.items()}
    control = results.pop("unmutated")
    assert control.returncode == 0, "the unmutated oracle must pass its pins:\n" + control.stdout[-3000:]
    survivors = [name for name, r in results.items() if r.returncode == 0]
    broken = {name: r.returncode for name, r in results.items() if r.returncode not in (0, 1)}
    assert not broken, f"pin runs that did not complete (exit codes): {broken}"
    assert not survivors, f"mutants no pin caught: {survivors}"
