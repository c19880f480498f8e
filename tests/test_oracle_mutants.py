"""Plant one plausible mistake at a time in a copy of the oracle (on the CPU) and check that
at least one pin catches it.  This is how the pins are shown to be sensitive: a dropped
term, a wrong sign or index, or a transposed operand anywhere in the oracle fails one."""
import os
import subprocess
import sys

import pytest

import oracle
from pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "sgqa_oracle.c")

# (name, original text, planted mistake)
MUTANTS = [
    ("mean-divides-by-B", "kb[j * P + p] = sum / (double)n;", "kb[j * P + p] = sum / (double)B;"),
    ("mean-drops-last-token", "for (int64_t s = first; s < first + n; ++s)\n                sum += widen_bf16(kp",
     "for (int64_t s = first; s < first + n - 1; ++s)\n                sum += widen_bf16(kp"),
    ("fused-mean-divides-by-B", "m[i] = sum / (double)n;", "m[i] = sum / (double)B;"),
    ("fused-weight-transposed", "acc += widen_bf16(wt[(int64_t)p * width + i]) * m[i];",
     "acc += widen_bf16(wt[(int64_t)i * P + p]) * m[i];"),
    ("fused-skips-first-token", "for (int64_t s = first; s < first + n; ++s)\n                    sum += widen_bf16(K",
     "for (int64_t s = first + 1; s < first + n; ++s)\n                    sum += widen_bf16(K"),
    ("own-block-scored", "return t / B;\n}\n\n/*\n * Block", "return t / B + 1;\n}\n\n/*\n * Block"),
    ("score-transposed-operand", "acc += widen_bf16(q[p]) * kb[j * P + p];",
     "acc += widen_bf16(q[p]) * kb[j * P + (P - 1 - p)];"),
    ("sort-ascending", "if (x->score > y->score)\n        return -1;",
     "if (x->score > y->score)\n        return 1;"),
    ("tie-prefers-high-index", "if (x->block < y->block)\n        return -1;",
     "if (x->block < y->block)\n        return 1;"),
    ("own-block-not-forced", "            row[count++] = (int32_t)c;\n            qsort",
     "            qsort"),
    ("small-case-drops-own", "for (int64_t j = 0; j <= c; ++j)", "for (int64_t j = 0; j < c; ++j)"),
    ("causal-excludes-self", "if (s <= t)", "if (s < t)"),
    ("scale-dropped", "z[s] = scale * dot;", "z[s] = dot;"),
    ("group-map-interleaved",
     "const int32_t g = h / heads_per_group;\n        double m = -INFINITY;\n        for (int64_t s = 0; s < n; ++s) {\n            double dot = 0.0;\n            for (int32_t i = 0; i < d; ++i)\n                dot += widen_bf16(q[h * d + i]) * krows[",
     "const int32_t g = h % Hkv;\n        double m = -INFINITY;\n        for (int64_t s = 0; s < n; ++s) {\n            double dot = 0.0;\n            for (int32_t i = 0; i < d; ++i)\n                dot += widen_bf16(q[h * d + i]) * krows["),
    ("backward-group-map-interleaved",
     "const int32_t g = h / heads_per_group;\n        double m = -INFINITY;\n        for (int64_t s = 0; s < n; ++s) {\n            double dot = 0.0;\n            for (int32_t i = 0; i < d; ++i)\n                dot += widen_bf16(q[h * d + i]) * widen_bf16(krows[",
     "const int32_t g = h % Hkv;\n        double m = -INFINITY;\n        for (int64_t s = 0; s < n; ++s) {\n            double dot = 0.0;\n            for (int32_t i = 0; i < d; ++i)\n                dot += widen_bf16(q[h * d + i]) * widen_bf16(krows["),
    ("key-is-value", "widen_bf16(q[h * d + i]) * krows[(s * Hkv + g) * d + i]",
     "widen_bf16(q[h * d + i]) * vrows[(s * Hkv + g) * d + i]"),
    ("backward-drops-D", "const double dz = P[s] * (dP[s] - Dsum);", "const double dz = P[s] * dP[s];"),
    ("backward-gate-derivative", "dgate[h] = go_a * sg * (1.0 - sg);", "dgate[h] = go_a * sg;"),
    ("backward-dv-ungated", "dvrows[(s * Hkv + g) * d + i] += P[s] * sg * widen_bf16(gout[h * d + i]);",
     "dvrows[(s * Hkv + g) * d + i] += P[s] * widen_bf16(gout[h * d + i]);"),
    ("backward-dq-unscaled", "dq[h * d + i] += scale * dz * widen_bf16(krows[(s * Hkv + g) * d + i]);",
     "dq[h * d + i] += dz * widen_bf16(krows[(s * Hkv + g) * d + i]);"),
    ("e4m3-bias-off-by-one", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    ("e4m3-truncates", "const double r = nearbyint(ldexp(a, 3 - E));", "const double r = floor(ldexp(a, 3 - E));"),
    ("e4m3-subnormal-edge", "if (a == 0.0 || E < -6)\n        E = -6;", "if (a == 0.0 || E < -7)\n        E = -7;"),
    ("fp8-scale-wrong-max", "float scale = amax / 448.0f;", "float scale = amax / 240.0f;"),
    ("gate-sign", "return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(x));"),
    ("no-normalisation", "out[h * d + i] = (acc / Z) * gate_factor;", "out[h * d + i] = acc * gate_factor;"),
    ("lse-drops-max", "lse[h] = m + log(Z);", "lse[h] = log(Z);"),
    ("softmax-no-max-shift", "z[s] = exp(z[s] - m);", "z[s] = exp(z[s]);"),
    ("window-one-too-wide", "int64_t first = t - W + 1;", "int64_t first = t - W;"),
    ("window-excludes-self", "for (int64_t s = first; s <= t; ++s)", "for (int64_t s = first; s < t; ++s)"),
]


RUNNER = """
import sys
sys.path.insert(0, {tests!r})
sys.path.insert(0, {root!r})
import oracle
from pins import ALL_PINS
lib = oracle.load({lib!r})
caught = []
for pin in ALL_PINS:
    try:
        pin(lib)
    except (AssertionError, ValueError, FloatingPointError):
        caught.append(pin.__name__)
print("CAUGHT", ",".join(caught))
"""


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, orig, bad, tmp_path):
    src = open(SRC).read()
    assert src.count(orig) == 1, f"mutation anchor for {name} not unique/present"
    mut_src = tmp_path / "mutant.c"
    mut_src.write_text(src.replace(orig, bad))
    lib_path = str(tmp_path / "libmutant.so")
    oracle.build(force=True, src=str(mut_src), out=lib_path)
    # each mutant runs in its own process: a planted mistake may also crash (e.g. write past
    # a buffer sized for the correct token count), which counts as caught
    tests_dir = os.path.dirname(os.path.abspath(__file__))
    code = RUNNER.format(tests=tests_dir, root=os.path.dirname(tests_dir), lib=lib_path)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        return  # the mutant crashed under the pins
    line = [l for l in r.stdout.splitlines() if l.startswith("CAUGHT")][-1]
    caught = [c for c in line[len("CAUGHT"):].strip().split(",") if c]
    assert caught, f"no pin caught mutant {name}"
