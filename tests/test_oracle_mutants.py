"""Planted mistakes in the oracle, on the CPU: each broken copy of oracle.c
must fail at least one pin.  This shows the pins would catch a dropped term,
a wrong sign or index, a transposed operand, a narrower accumulator, a
reordered combine, a flipped tie rule, an unstable grouping or a swapped
operand in the oracle itself.
"""
import os
import subprocess
import sys

import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text to replace, replacement, which occurrence: 0 = first)
MUTANTS = [
    ("drop_last_term", "for (long k = 0; k < K; ++k) {", "for (long k = 0; k < K - 1; ++k) {", 0),
    ("wrong_sign", "        s += prod;", "        s -= prod;", 0),
    ("no_abs", "abs_s += fabs(prod);", "abs_s += prod;", 0),
    ("fp32_accumulator", "double s = 0.0, abs_s = 0.0;", "float s = 0.0f; double abs_s = 0.0;", 0),
    ("ignore_row_list", "long i = rows ? rows[r] : r;", "long i = r < M ? r : 0;", 0),
    ("weight_row_from_x_index", "const uint16_t *wn = w + n * K;", "const uint16_t *wn = w + (n % (M > 0 ? M : 1)) * K;", 0),
    ("i64_squares_x", "(int64_t)bf16_to_f64(w[n * K + k])", "(int64_t)bf16_to_f64(x[i * K + k])", 0),
    ("grouped_inclusive_end", "(offsets[e] <= i && i < offsets[e + 1])", "(offsets[e] <= i && i <= offsets[e + 1])", 0),
    ("grouped_expert_stride", "w + (e * N + n) * K", "w + n * K", 0),
    ("fold_reversed",
     "volatile float t = parts[j];\n        for (long s = 1; s < S; ++s)\n            t = t + parts[s * count + j];",
     "volatile float t = parts[(S - 1) * count + j];\n        for (long s = S - 2; s >= 0; --s)\n            t = t + parts[s * count + j];", 0),
    ("fold_in_fp64", "volatile float t = parts[j];", "volatile double t = parts[j];", 0),
    ("topk_ties_to_higher_id", "if (best < 0 || l[e] > l[best])", "if (best < 0 || l[e] >= l[best])", 0),
    ("topk_weight_sign", "z[j] = exp((double)l[id[j]] - (double)l[id[0]]);",
     "z[j] = exp((double)l[id[0]] - (double)l[id[j]]);", 0),
    ("permute_unstable",
     "for (long t = 0; t < T; ++t)\n            for (long j = 0; j < k; ++j)\n                if (ids[t * k + j] == e) {",
     "for (long t = T - 1; t >= 0; --t)\n            for (long j = 0; j < k; ++j)\n                if (ids[t * k + j] == e) {", 0),
    ("permute_offset_index", "offsets[ids[i] + 1] += 1;", "offsets[ids[i]] += 1;", 0),
    ("swiglu_sigmoid_sign", "a[r * I + i] = g / (1.0 + exp(-g)) * u;", "a[r * I + i] = g / (1.0 + exp(g)) * u;", 0),
    ("swiglu_gate_up_swapped", "double g = h[r * 2 * I + i];", "double g = h[r * 2 * I + I + i];", 0),
    ("combine_drops_last_expert", "for (long j = 0; j < k; ++j) {\n                double p = (double)w",
     "for (long j = 0; j < k - 1; ++j) {\n                double p = (double)w", 0),
    ("combine_ignores_weight", "double p = (double)w[t * k + j] * ", "double p = 1.0 * ", 0),
    ("rmsnorm_no_eps", "double inv = 1.0 / sqrt(ms[t] + eps);", "double inv = 1.0 / sqrt(ms[t]);", 0),
    ("rmsnorm_sum_not_mean", "ms[t] = s / (double)H;", "ms[t] = s;", 0),
    ("rmsnorm_no_gain", "y[t * H + h] = bf16_to_f64(x[t * H + h]) * bf16_to_f64(g[h]) * inv;",
     "y[t * H + h] = bf16_to_f64(x[t * H + h]) * inv;", 0),
    ("attn_kv_head_modulo", "kvh = h / G;", "kvh = h % Hkv;", 0),
    ("attn_no_scale", "const double e = exp(s * scale - smax);", "const double e = exp(s - smax);", 0),
    ("attn_drops_last_key", "n = seq_start[b + 1] - t0;", "n = seq_start[b + 1] - t0 - (seq_start[b + 1] > t0);", 0),
    ("attn_values_from_keys", "const uint16_t *vt = v + ((t0 + t) * Hkv + kvh) * D;",
     "const uint16_t *vt = k + ((t0 + t) * Hkv + kvh) * D;", 0),
]


def _mutate(text, old, new, occurrence):
    pos = -1
    for _ in range(occurrence + 1):
        pos = text.index(old, pos + 1)
    return text[:pos] + new + text[pos + len(old):]


# Runs every pin against one compiled mutant in a child process: a planted
# mistake may write out of bounds (a shifted offset table does), and that
# must not corrupt the test runner's heap.  Prints the pins that failed.
CHILD = r"""
import sys
sys.path[:0] = sys.argv[3:]
import oracle
from oracle_pins import ALL_PINS
lib = oracle.open_library(sys.argv[1])
failed = []
for pin in ALL_PINS:
    try:
        pin(lib=lib)
    except (AssertionError, ValueError):
        failed.append(pin.__name__)
print("FAILED_PINS", len(failed), " ".join(failed))
"""


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new, occ):
    text = open(SRC).read()
    assert old in text, "mutation site vanished: " + name
    src = tmp_path / ("oracle_%s.c" % name)
    src.write_text(_mutate(text, old, new, occ))
    so = oracle.compile_source(str(src), str(tmp_path / ("lib%s.so" % name)))
    here = os.path.dirname(os.path.abspath(__file__))
    res = subprocess.run([sys.executable, "-c", CHILD, so, name, here, os.path.dirname(here)],
                         capture_output=True, text=True, timeout=300)
    lines = [l for l in res.stdout.splitlines() if l.startswith("FAILED_PINS")]
    if lines:  # the pins ran to the end (the process may still crash on exit)
        assert int(lines[-1].split()[1]) > 0, "no pin caught the planted mistake " + name
    else:
        assert res.returncode < 0, res.stderr[-2000:]  # a pin run crashed: caught
