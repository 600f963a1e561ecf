"""The oracle's pins must catch plausible mistakes.

Each case copies the oracle source, plants one mistake by a textual edit (a
wrong window edge, a dropped diagonal, a wrong head grouping, a wrong sign, a
sum over the wrong axis, a reversed tie rule, ...), builds the copy on the CPU
and checks that at least one pin fails on it.  The oracle itself is never
edited.
"""
import math
import os
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle

MUTANTS = {
    "window_edge": [("if (j + window <= i)", "if (j + window < i)")],
    "no_diagonal": [("const int64_t n = i + 1;", "const int64_t n = i > 0 ? i : 1;")],
    "interleaved_groups": [("(b * Hq + h * G + gg) * S * D", "(b * Hq + gg * Hkv + h) * S * D"),
                           ("const int64_t g = h * G + gg;", "const int64_t g = gg * Hkv + h;")],
    "no_scale": [("logit[j] *= scale;", "logit[j] *= 1.0;")],
    "exp_sign": [("logit[j] = std::exp(logit[j] - m);", "logit[j] = std::exp(m - logit[j]);")],
    "row_sum_not_column": [("col[j] += p[j];", "col[i] += p[j];")],
    "dropped_partition": [("for (int64_t it = 0; it < n_items; ++it) acc",
                           "for (int64_t it = 1; it < n_items; ++it) acc")],
    "ties_to_higher_index": [("return a.second < b.second;", "return a.second > b.second;")],
    "eligible_skips_first": [("for (int64_t j = n_sink; j < S - window; ++j) elig",
                              "for (int64_t j = n_sink + 1; j < S - window; ++j) elig")],
    "no_sinks": [("for (int64_t j = 0; j < std::min(n_sink, S); ++j) kept[j] = 1;", "")],
    "lse_without_max": [("return {m + std::log(z), rowsum};", "return {std::log(z), rowsum};")],
}


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _widen(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _pins(lib):
    """A compact set of the oracle pins, parameterised by library.  Returns
    the list of failed pin names."""
    failed = []

    def check(name, fn):
        try:
            if not fn():
                failed.append(name)
        except Exception:  # an exception (bad rc, nan compare) is a failure too
            failed.append(name)

    rng = np.random.default_rng(99)
    S, D, w = 48, 64, 5

    def uniform():
        kb = _bf16(rng.standard_normal((1, 1, S, D)))
        qb = np.zeros((1, 2, S, D), np.uint16)
        out = oracle.future_mass(qb, kb, w, lib=lib)
        HS = sum(Fraction(1, m) for m in range(1, S + 1))
        exp = [float(2 * (HS - sum(Fraction(1, m) for m in range(1, j + w + 1)))) if j + w < S else 0.0
               for j in range(S)]
        return (np.allclose(out["lse"][0], np.log(np.arange(1, S + 1))[None], atol=1e-12)
                and np.allclose(out["mass"][0, 0], exp, rtol=1e-12, atol=1e-15))

    def brute():
        qb = _bf16(rng.standard_normal((1, 4, S, D)) * 1.5)
        kb = _bf16(rng.standard_normal((1, 2, S, D)) * 1.5)
        out = oracle.future_mass(qb, kb, w, lib=lib)
        q, k = _widen(qb), _widen(kb)
        mass = np.zeros((1, 2, S))
        lse = np.zeros((1, 4, S))
        ii, jj = np.arange(S)[:, None], np.arange(S)[None, :]
        for g in range(4):
            L = np.where(jj <= ii, q[0, g] @ k[0, g // 2].T / math.sqrt(D), -np.inf)
            lse[0, g] = scipy.special.logsumexp(L, axis=1)
            mass[0, g // 2] += np.where(ii >= jj + w, scipy.special.softmax(L, axis=1), 0).sum(0)
        return np.allclose(out["mass"], mass, rtol=1e-10) and np.allclose(out["lse"], lse, rtol=1e-12)

    def select():
        m = np.round(rng.random((1, 2, 60)) * 6) / 6
        keep = oracle.select(m, 7, 4, 9, lib=lib)
        for h in range(2):
            elig = sorted(range(4, 53), key=lambda j: (-m[0, h, j], j))[:9]
            exp = sorted(set(range(4)) | set(range(53, 60)) | set(elig))
            if keep[0, h].tolist() != exp:
                return False
        return True

    def needle():
        Sn, js = 40, 11
        q = np.ones((1, 1, Sn, D), np.float32)
        k = rng.standard_normal((1, 1, Sn, D)).astype(np.float32) * 0.25
        k[0, 0, js] = 8.0
        mass = oracle.future_mass(_bf16(q), _bf16(k), 3, lib=lib)["mass"]
        return abs(mass[0, 0, js] - (Sn - js - 3)) < 1e-9

    check("uniform_closed_form", uniform)
    check("matrix_brute_force", brute)
    check("select_brute_force", select)
    check("needle", needle)
    return failed


def test_unmodified_oracle_passes_compact_pins():
    assert _pins(oracle.load()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    src = open(oracle._SRC).read()
    for old, new in MUTANTS[name]:
        assert old in src, f"mutant {name}: pattern not found (oracle source changed?)"
        src = src.replace(old, new)
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, "mutant.cpp")
        with open(path, "w") as f:
            f.write(src)
        lib = oracle.load(oracle.build(src=path, out=os.path.join(td, f"lib_{name}.so")))
        failed = _pins(lib)
    assert failed, f"planted mistake '{name}' passed every pin"
