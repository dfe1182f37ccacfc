"""Planted mistakes in the oracle, on the CPU: each mutant below is a copy of
the oracle's C source with one plausible mistake (a dropped term, a wrong
sign, index or bound), compiled on its own.  The pin suite must fail on every
one of them, which shows the pins constrain each step of the oracle."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "no_softmax_scale": ("x[i] = acc / scale;", "x[i] = acc;"),
    "replace_not_accumulate": ("c->snew[i] = prm->current_score ? inc : c->s[i] + inc;",
                               "c->snew[i] = inc;"),
    "tova_accumulates": ("c->snew[i] = prm->current_score ? inc : c->s[i] + inc;",
                         "c->snew[i] = c->s[i] + inc;"),
    "rotation_sign": ("float y1 = a - b;", "float y1 = a + b;"),
    "rotation_direction": ("float s = (float)sin(theta);", "float s = (float)sin(-theta);"),
    "frequency_index": ("-(2.0 * (double)j) / (double)d", "-(2.0 * (double)(j + 1)) / (double)d"),
    "delta_sign": ("int64_t delta = (int64_t)j - (int64_t)c->p[src];",
                   "int64_t delta = (int64_t)c->p[src] - (int64_t)j;"),
    "new_row_not_remapped": ("c->p[n] = c->next_pos;", "c->p[n] = n;"),
    "tie_to_highest": ("if (e < 0 || key < best) {", "if (e < 0 || key <= best) {"),
    "sinks_evictable": ("for (int32_t i = prm->n_sink; i <= last; ++i) {",
                        "for (int32_t i = 0; i <= last; ++i) {"),
    "new_row_protected": ("const int32_t last = n - prm->recent;",
                          "const int32_t last = n - prm->recent - 1;"),
    "recent_ignored": ("const int32_t last = n - prm->recent;", "const int32_t last = n;"),
    "recent_window_one_short": ("const int32_t last = n - prm->recent;",
                                "const int32_t last = n - prm->recent + (prm->recent > 0);"),
    "recent_not_validated": ("prm->budget <= prm->n_sink + prm->recent ||",
                             "prm->budget <= prm->n_sink ||"),
    "evict_one_early": ("if (n + 1 > prm->budget) {", "if (n + 1 >= prm->budget) {"),
    "tau_pos_after_increment": ("prm->anneal_steps, c->pos) : 0.0f;",
                                "prm->anneal_steps, c->pos + 1) : 0.0f;"),
    "gumbel_sign": ("return (float)(-log(-log(u)));", "return (float)(log(-log(u)));"),
    "splitmix_shift": ("return z ^ (z >> 31);", "return z ^ (z >> 30);"),
    "values_not_moved": ("copy_row(c->v + (size_t)j * d, c->v + (size_t)src * d, d);", ""),
    "gumbel_not_moved": ("c->g[j] = c->g[src];", ""),
    "scores_not_moved": ("c->s[j] = c->s[src];", ""),
    "pyramid_top": ("double hi = 2.0 * (double)avg_budget - lo;",
                    "double hi = beta * (double)avg_budget;"),
    "f16_ties_away": ("double r = rint(a / q) * q;", "double r = floor(a / q + 0.5) * q;"),
    "tau_no_clamp": ("int64_t t = pos < (int64_t)anneal_steps ? pos : (int64_t)anneal_steps;",
                     "int64_t t = pos;"),
}


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "kve_oracle.c")).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/absent"
    mutated = tmp_path / "kve_oracle.c"
    mutated.write_text(src.replace(old, new))
    hdr = tmp_path / "kve_oracle.h"
    hdr.write_text(open(os.path.join(ROOT, "oracle", "kve_oracle.h")).read())
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", *oracle.GCC_FLAGS, "-w", "-o", str(lib), str(mutated), "-lm"],
                   check=True)
    env = dict(os.environ, KVE_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pin suite:\n{r.stdout[-2000:]}"
