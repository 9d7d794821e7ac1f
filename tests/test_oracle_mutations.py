"""The oracle's pins catch plausible mistakes (CPU only).

Each mutant below is a copy of oracle/oracle.c with one deliberate mistake
planted by a textual replacement: a flipped sign, a wrong index, a dropped
term, a changed constant, a reordered sum.  It is compiled with the oracle's
own flags, and the oracle's pin tests are run against it in a subprocess
(through the loader's library override).  Every mutant must fail at least one
pin; the unaltered copy, run the same way, must pass them all.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

from oracle import LIB_ENV
from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = [os.path.join(ROOT, "tests", f) for f in (
    "test_oracle_codecs.py", "test_oracle_steps.py", "test_oracle_ops.py",
    "test_oracle_variants.py", "test_oracle_indexer.py")]

# (name, text in oracle.c (must occur exactly once), replacement)
MUTANTS = [
    ("inverse rotation: wrong sign of e*s",
     "y[2 * k + 1] = oc - es;", "y[2 * k + 1] = oc + es;"),
    ("forward rotation: wrong sign of o*s",
     "y[2 * k] = ec - os;", "y[2 * k] = ec + os;"),
    ("sin taken from the next column",
     "float s = cs_row[HALF_ROPE + k - NOPE_DIM / 2];",
     "float s = cs_row[HALF_ROPE + (k - NOPE_DIM / 2 + 1) % HALF_ROPE];"),
    ("cos read from the sin half",
     "float c = cs_row[k - NOPE_DIM / 2];", "float c = cs_row[HALF_ROPE + k - NOPE_DIM / 2];"),
    ("first rotated pair skipped",
     "for (k = NOPE_DIM / 2; k < HEAD_DIM / 2; ++k) {",
     "for (k = NOPE_DIM / 2 + 1; k < HEAD_DIM / 2; ++k) {"),
    ("scale divisor 447", "s = m / E4M3_MAX;", "s = m / 447.0f;"),
    ("amax floor dropped", "    if (eps > m) m = eps;\n    if (scale_fmt", "    if (scale_fmt"),
    ("e4m3 ties away from zero",
     "(frac == 0.5f && fmodf(fl, 2.0f) == 1.0f)", "(frac == 0.5f)"),
    ("NaN encoded as 448", "return (uint8_t)((sign << 7) | 0x7Fu);",
     "return (uint8_t)((sign << 7) | 0x7Eu);"),
    ("bf16 rounds half up",
     "if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;",
     "if (rest >= 0x8000u) keep += 1u;"),
    ("pow2 ceiling always rounds up", "  if (u & 0x7FFFFFu) k += 1;", "  k += 1;"),
    ("UE8M0 exponent bytes in reverse order",
     "word |= (uint32_t)(k + 127) << (8 * b);", "word |= (uint32_t)(k + 127) << (8 * (3 - b));"),
    ("RMSNorm mean over 511", "float mean = ss / 512.0f;", "float mean = ss / 511.0f;"),
    ("RMSNorm eps dropped", "float r = 1.0f / sqrtf(mean + eps);", "float r = 1.0f / sqrtf(mean);"),
    ("RMSNorm weight reversed", "v * orc_bf16_to_f32(weight[d])",
     "v * orc_bf16_to_f32(weight[HEAD_DIM - 1 - d])"),
    ("RMSNorm squares summed right to left",
     "  float ss = x[0] * x[0];\n  for (d = 1; d < n; ++d) ss = ss + x[d] * x[d];",
     "  float ss = x[n - 1] * x[n - 1];\n"
     "  for (d = n - 2; d >= 0; --d) ss = ss + x[d] * x[d];"),
    ("pairwise sum split at a quarter",
     "return sum_squares_pairwise(x, n / 2) + sum_squares_pairwise(x + n / 2, n - n / 2);",
     "return sum_squares_pairwise(x, (n + 2) / 4) + sum_squares_pairwise(x + (n + 2) / 4, "
     "n - (n + 2) / 4);"),
    ("pairwise sum taken left to right",
     "return sum_squares_pairwise(x, n / 2) + sum_squares_pairwise(x + n / 2, n - n / 2);",
     "return sum_squares_pairwise(x, n - 1) + x[n - 1] * x[n - 1];"),
    ("IRQ scale index transposed", "(j * NBLOCK + b) * sc_stride_block",
     "(b * heads_per_group + j) * sc_stride_block"),
    ("IRQ codes at the token-major column", "out[g * out_stride_group + t * out_stride_token + "
     "j * HEAD_DIM + d] = codes[d];", "out[g * out_stride_group + t * out_stride_token + "
     "(j ^ 1) % heads_per_group * HEAD_DIM + d] = codes[d];"),
    ("QNR pad heads not zero", "for (d = 0; d < HEAD_DIM; ++d) dst[d] = 0;",
     "for (d = 0; d < HEAD_DIM; ++d) dst[d] = 0x8000;"),
    ("QNR inverse rotation",
     "      orc_rope_head(y, z, row, 0);\n      for (d = 0; d < HEAD_DIM; ++d) dst[d]",
     "      orc_rope_head(y, z, row, 1);\n      for (d = 0; d < HEAD_DIM; ++d) dst[d]"),
    ("q FP8 pad head not a zero head", "        memset(z, 0, sizeof z);",
     "        memset(z, 0, sizeof z);\n        z[0] = 1.0f;"),
    ("q FP8 quant eps doubled", "qepsf = (float)quant_eps;", "qepsf = 2.0f * (float)quant_eps;"),
    ("KVI 512-byte record stride", "(s % cache_block_size) * RECORD_BYTES;",
     "(s % cache_block_size) * HEAD_DIM;"),
    ("KVI negative slot written to slot 0",
     "    if (s < 0) continue;\n    load_head(kv + t * kv_stride_token, x);\n"
     "    orc_rope_head(x, y, cos_sin_cache + positions[t] * ROPE_DIM, 0);\n    orc_quant_head",
     "    if (s < 0) s = 0;\n    load_head(kv + t * kv_stride_token, x);\n"
     "    orc_rope_head(x, y, cos_sin_cache + positions[t] * ROPE_DIM, 0);\n    orc_quant_head"),
    ("KVI scale bytes in reverse block order", "memcpy(rec + HEAD_DIM + 4 * b, &sf[b], 4);",
     "memcpy(rec + HEAD_DIM + 4 * b, &sf[3 - b], 4);"),
    ("inv_rope_bf16 forward rotation",
     "      orc_rope_head(x, y, row, 1);\n      for (d = 0; d < HEAD_DIM; ++d) dst[d]",
     "      orc_rope_head(x, y, row, 0);\n      for (d = 0; d < HEAD_DIM; ++d) dst[d]"),
    ("inv_rope_bf16 low bit flipped", "dst[d] = orc_f32_to_bf16(y[d]);",
     "dst[d] = orc_f32_to_bf16(y[d]) ^ (d == 5);"),
    ("kv bf16 cache rows at a 512-element stride", "cache[s * cache_stride_token + d]",
     "cache[s * HEAD_DIM + d]"),
    ("kv bf16 cache inverse rotation",
     "ROPE_DIM, 0);\n    for (d = 0; d < HEAD_DIM; ++d) cache[",
     "ROPE_DIM, 1);\n    for (d = 0; d < HEAD_DIM; ++d) cache["),
    ("indexer rotate-half sign", "y[i] = orc_bf16_to_f32(orc_f32_to_bf16(a - b));",
     "y[i] = orc_bf16_to_f32(orc_f32_to_bf16(a + b));"),
    ("indexer bf16 round trip dropped",
     "y[i + 32] = orc_bf16_to_f32(orc_f32_to_bf16(d + e));", "y[i + 32] = d + e;"),
    ("indexer weight fold reassociated",
     "*w_out = ((w * *q_scale) * softmax_scale) * head_scale;",
     "*w_out = w * (*q_scale * (softmax_scale * head_scale));"),
]


def _build(src_text, out_dir, tag):
    src = os.path.join(out_dir, f"oracle_{tag}.c")
    lib = os.path.join(out_dir, f"liboracle_{tag}.so")
    with open(src, "w") as f:
        f.write(src_text)
    # the oracle's flags, less -Werror: a planted mistake may leave a
    # parameter unused
    flags = [f for f in oracle_build.CFLAGS if f != "-Werror"]
    cmd = ["gcc", *flags, src, "-o", lib, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, f"{tag}: the mutant does not compile:\n{res.stderr}"
    return lib


def _pins_pass(lib):
    env = dict(os.environ, **{LIB_ENV: lib})
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          *PINS], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=600)
    return res.returncode == 0, res.stdout[-600:]


@pytest.mark.slow
def test_every_planted_mistake_fails_a_pin(tmp_path):
    with open(oracle_build.SRC) as f:
        base = f.read()
    jobs = [("control", base)]
    for i, (name, old, new) in enumerate(MUTANTS):
        assert base.count(old) == 1, f"mutant '{name}': its text occurs {base.count(old)} times"
        jobs.append((f"m{i:02d}", base.replace(old, new)))
    libs = {tag: _build(text, str(tmp_path), tag) for tag, text in jobs}
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(workers) as ex:
        results = dict(zip(libs, ex.map(_pins_pass, libs.values())))
    ok, out = results.pop("control")
    assert ok, f"the unaltered oracle fails its pins through the override:\n{out}"
    survivors = [MUTANTS[int(tag[1:])][0] for tag, (passed, _) in results.items() if passed]
    print(f"[mutants] {len(MUTANTS) - len(survivors)}/{len(MUTANTS)} caught")
    assert not survivors, f"mutants no pin catches: {survivors}"
