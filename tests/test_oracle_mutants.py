"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a temporary copy of the oracle's C source
(a dropped term, a wrong sign or index, a transposed operand, a wrong tie
rule, a wrong rounding, ...), builds that copy, routes the oracle module to
it and runs every pin of tests/test_oracle_pins.py.  At least one pin must
fail for every planted mistake; the unmodified source must pass them all.
Every mutation keeps all memory accesses in bounds, so a broken copy can
only compute wrong numbers.
"""
import inspect
import os

import pytest

import oracle
from oracle import build as obuild
from tests import test_oracle_pins as pins

SRC = open(obuild.SRC).read()

# (name, text in the source, replacement): each text occurs exactly once
MUTANTS = [
    ("distance is not squared", "                D += t * t;\n            }\n            if (D < best)",
     "                D += fabs(t);\n            }\n            if (D < best)"),
    ("sign of the difference", "                double t = x[k] - c[k];",
     "                double t = x[k] + c[k];"),
    ("last coordinate dropped", "            for (int64_t k = 0; k < d; ++k) {\n                double t = x[k] - c[k];",
     "            for (int64_t k = 0; k < d - 1; ++k) {\n                double t = x[k] - c[k];"),
    ("centroid rows transposed", "            const double *c = Cb + j * d;",
     "            const double *c = Cb + j;"),
    ("ties go to the largest index", "            if (D < best) {", "            if (D <= best) {"),
    ("second-nearest distance not kept", "            } else if (D < second) {", "            } else if (0) {"),
    ("weights dropped from the sums", "            for (int64_t k = 0; k < d; ++k) S[j * d + k] += wi * x[k];",
     "            for (int64_t k = 0; k < d; ++k) S[j * d + k] += x[k];"),
    ("weight sum counts points", "            W[j] += wi;", "            W[j] += 1.0;"),
    ("empty cluster reset to zero", "                cn[k] = Nj[j] > 0 ? (float)(S[j * d + k] / W[j]) : co[k];",
     "                cn[k] = Nj[j] > 0 ? (float)(S[j * d + k] / W[j]) : 0.0f;"),
    ("first point not counted", "            Nj[j] += 1;", "            Nj[j] += (i > 0);"),
    ("last point left out of the update", "        for (int64_t i = 0; i < N; ++i) {\n            int64_t j = labels[b * N + i];\n            double wi",
     "        for (int64_t i = 0; i + 1 < N; ++i) {\n            int64_t j = labels[b * N + i];\n            double wi"),
    ("rounding truncates", "        if (r > half || (r == half && (q & 1ull))) q += 1ull;", "        if (0) q += 1ull;"),
    ("rounding ties away from zero", "        if (r > half || (r == half && (q & 1ull))) q += 1ull;",
     "        if (r >= half) q += 1ull;"),
    ("subnormal decode exponent", "        v = ldexp((double)m, (1 - bias) - man_bits);",
     "        v = ldexp((double)m, (0 - bias) - man_bits);"),
    ("fit skips rounding the centroids", "                Ch[i] = oracle_decode_one(cbits[i], dtype);",
     "                Ch[i] = (double)C_out[i];"),
    ("objective ignores the weights", "                    J += (Wd ? Wd[b * N + i] : 1.0) * d1_out[b * N + i];",
     "                    J += d1_out[b * N + i];"),
    ("objective of the previous centroids", "                J_out[b * n_iter + t] = J;",
     "                J_out[b * n_iter + t] = t > 0 ? J_out[b * n_iter + t - 1] : J;"),
    ("optimum: running scatter ignores the weights", "                        sse += wi * delta * (xi - mean_n);",
     "                        sse += delta * (xi - mean_n);"),
    ("optimum: running mean update unweighted", "                        const double mean_n = mean + wi * delta / Wn;",
     "                        const double mean_n = mean + delta / Wn;"),
    ("optimum: previous prefix one point too long", "                        const double cand = D[(k - 1) * (N + 1) + i] + sse;",
     "                        const double cand = D[(k - 1) * (N + 1) + i + 1] + sse;"),
    ("optimum: ties go to the latest cut", "                        if (cand <= best) {", "                        if (cand < best) {"),
    ("optimum: last run starts one point late", "        bound[K] = N;\n            for (int64_t k = K; k >= 1; --k) bound[k - 1] = cut[k * (N + 1) + bound[k]];",
     "        bound[K] = N;\n            for (int64_t k = K; k >= 1; --k) bound[k - 1] = cut[k * (N + 1) + bound[k]] + (k == K);"),
    ("optimum: means not weighted", "                    swx += ws[p] * xs[p];", "                    swx += xs[p];"),
    ("optimum: runs numbered from the top", "                    labels_out[b * N + s[p].i] = (int32_t)k;",
     "                    labels_out[b * N + s[p].i] = (int32_t)(K - 1 - k);"),
    ("e-means: step weights swapped", "                    S[j * d + c] = (1.0 - a) * S[j * d + c] + a * s[j * d + c];",
     "                    S[j * d + c] = a * S[j * d + c] + (1.0 - a) * s[j * d + c];"),
    ("e-means: counts accumulate without decay", "                Nc[j] = (1.0 - a) * Nc[j] + a * n[j];",
     "                Nc[j] = Nc[j] + n[j];"),
    ("e-means: no final mean", "            if (G[j] > 0.0)\n", "            if (0)\n"),
    ("e-means: donor not halved", "                Nc[k] *= 0.5;", "                Nc[k] *= 1.0;"),
    ("e-means: donor drawn from the top", "                const double target = (double)uniforms[t * K + j] * P[K];",
     "                const double target = (1.0 - (double)uniforms[t * K + j]) * P[K];"),
    ("e-means: schedule floor ignored", "alpha0 * floor_frac +\n", "alpha0 * 0.0 +\n"),
    ("e-means: deadness re-read after each split", "                if (!dead[j]) continue;",
     "                if (!(Nc[j] < dead_below)) continue;"),
]


def _pin_functions():
    out = []
    for name, fn in sorted(vars(pins).items()):
        if name.startswith("test_") and callable(fn):
            params = list(inspect.signature(fn).parameters)
            assert params == ["orc"], f"{name} takes {params}"
            out.append((name, fn))
    return out


def _failing_pins(lib_path):
    failed = []
    with oracle.using_library(lib_path):
        for name, fn in _pin_functions():
            try:
                fn(oracle)
            except Exception:  # an assertion, or a check that cannot even run
                failed.append(name)
    return failed


def _build(tmp_path, text, tag):
    src = os.path.join(tmp_path, f"oracle_{tag}.c")
    with open(src, "w") as f:
        f.write(text)
    return obuild.compile_source(src, os.path.join(tmp_path, f"liboracle_{tag}.so"))


def test_unmodified_source_passes_every_pin(tmp_path):
    assert _failing_pins(_build(str(tmp_path), SRC, "clean")) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    assert SRC.count(old) == 1, f"mutation site of '{name}' not unique"
    failed = _failing_pins(_build(str(tmp_path), SRC.replace(old, new), "mut"))
    assert failed, f"no pin fails when the oracle has this mistake: {name}"
