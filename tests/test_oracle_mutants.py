"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle/bsa_oracle.c, applies one small textual mutation of
the kind a careless implementation could make (wrong comparison, dropped term,
wrong index, swapped head mapping, ...), builds it with gcc into a temporary
library and runs tests/test_oracle_pins.py against that library.  The pins
must fail.  Everything runs on the CPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "bsa_oracle.c")

MUTANTS = {
    "envelope-picks-min": ("term = x > y ? x : y;", "term = x < y ? x : y;"),
    "envelope-drops-kmin": ("double x = q[d] * kmin[d], y = q[d] * kmax[d];",
                            "double x = 0.0 * kmin[d], y = q[d] * kmax[d];"),
    "centroid-wrong-count": ("cen[o + d] = sum / (double)(e - s);", "cen[o + d] = sum / (double)(e - s + 1);"),
    "page-interval-short": ("*e = *s + c->page_size < L ? *s + c->page_size : L;",
                            "*e = *s + c->page_size - 1 < L ? *s + c->page_size - 1 : L;"),
    "tie-break-reversed": ("return (a->i > b->i) - (a->i < b->i);", "return (a->i < b->i) - (a->i > b->i);"),
    "group-sum-not-max": ("if (s > best) best = s;\n                    if (den > best_den)",
                          "best = (best == -INFINITY ? 0.0 : best) + s;\n                    if (den > best_den)"),
    "ratio-ceil": ("int K = (int)floor((double)n * ratio);", "int K = (int)ceil((double)n * ratio);"),
    "eos-wrong-page": ("if (n > 0 && eos && !taken[n - 1]) { taken[n - 1] = 1; keep[m++] = n - 1; }",
                       "if (n > 1 && eos && !taken[n - 2]) { taken[n - 2] = 1; keep[m++] = n - 2; }"),
    "token-budget-overshoot": ("if (total + len[order[i].i] > tokens) break;",
                               "if (total > tokens) break;"),
    "softmax-scale-dropped": ("logit[t] = s * scale;", "logit[t] = s;"),
    "gqa-head-mapping": ("int h = j / g, L = c->seq_lens[b];", "int h = j % Hkv, L = c->seq_lens[b];"),
    "sigma-wrong-rank": ("sk1 = order[k - 1].s, sk = order[k].s;", "sk1 = order[k - 1].s, sk = order[k + 1 < n ? k + 1 : k].s;"),
    "sigma-inverted": ("sg = (s0 == sk) ? 0.0 : (sk1 - sk) / (s0 - sk);", "sg = (s0 == sk) ? 0.0 : (s0 - sk1) / (s0 - sk);"),
    "quantile-position": ("double pos = (m - 1) * p;", "double pos = m * p;"),
    "trigger-non-strict": ("triggered[t] = eligible[t] && (sigma_bar[t] < *tau);",
                           "triggered[t] = eligible[t] && (sigma_bar[t] <= *tau);"),
    "sigma-bar-sum": ("sigma_bar[t] = acc / num_kv_heads;", "sigma_bar[t] = acc;"),
    "sigma-bar-max-over-heads": ("acc += sigma[(int64_t)t * num_kv_heads + h];\n        sigma_bar[t] = acc / num_kv_heads;",
                                 "acc = fmax(acc, sigma[(int64_t)t * num_kv_heads + h]);\n        sigma_bar[t] = acc;"),
    "sigma-bar-first-head": ("sigma_bar[t] = acc / num_kv_heads;", "sigma_bar[t] = sigma[(int64_t)t * num_kv_heads];"),
    "quantile-over-all-tiles": ("if (eligible[t]) elig_vals[m++] = sigma_bar[t];", "elig_vals[m++] = sigma_bar[t];"),
    "expansion-swapped": ("int keep = triggered[t] ? width : k;", "int keep = triggered[t] ? k : width;"),
    "tile-diagonal-hidden": ("int v = last / block_size + 1;", "int v = last / block_size;"),
    "causal-leak": ("if (p > r) break;", "if (p > r + 1) break;"),
    "tile-score-first-row": ("for (int r = r0; r < r1; ++r)", "for (int r = r0; r < r0 + 1; ++r)"),
    "bos-forced-second-page": ("if (n > 0 && bos && !taken[0]) { taken[0] = 1; keep[m++] = 0; }",
                               "if (n > 1 && bos && !taken[1]) { taken[1] = 1; keep[m++] = 1; }"),
    "kmax-skips-last-token": ("if (x > hi) hi = x;", "if (x > hi && t + 1 < e) hi = x;"),
    "decode-skips-first-selected": ("for (int i = 0; i < cnt; ++i) {\n                    int s, e;",
                                    "for (int i = 1; i < cnt; ++i) {\n                    int s, e;"),
    "expansion-unsorted": ("qsort(dst, keep, sizeof(int32_t), int_cmp);", ""),
    "sentinel-zero": ("for (int i = keep; i < width; ++i) dst[i] = -1;", "for (int i = keep; i < width; ++i) dst[i] = 0;"),
}


def _build(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mutated = tmp_path / f"{name}.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / f"lib{name}.so"
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC", "-o",
                           str(lib), str(mutated), "-lm"])
    return lib


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(tmp_path, name):
    old, new = MUTANTS[name]
    lib = _build(tmp_path, name, old, new)
    env = dict(os.environ, BSA_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
