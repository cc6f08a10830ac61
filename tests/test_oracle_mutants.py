"""The pins catch plausible mistakes: each test plants one mistake in a copy of the oracle's
C source (on the CPU), builds it, and checks that the pin suite fails against it."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "condensate_oracle.c")

MUTANTS = {
    "window_one_short": ("(i - p->W + 1 > 0) ? i - p->W + 1 : 0", "(i - p->W + 2 > 0) ? i - p->W + 2 : 0"),
    "candidates_overlap_window": ("const int64_t r_last = i - p->W;", "const int64_t r_last = i - p->W + 1;"),
    "topk_over_all_positions": ("const int64_t n_r = r_last >= 1 ? r_last : 0;", "const int64_t n_r = i;"),
    "tie_break_reversed": ("return (a->j < b->j) ? -1 : (a->j > b->j);", "return (a->j > b->j) ? -1 : (a->j < b->j);"),
    "ascending_sort": ("if (a->s > b->s) return -1;\n    if (a->s < b->s) return 1;",
                       "if (a->s < b->s) return -1;\n    if (a->s > b->s) return 1;"),
    "scale_dropped": ("return acc * (1.0 / sqrt((double)p->d));", "return acc;"),
    "scale_by_d": ("return acc * (1.0 / sqrt((double)p->d));", "return acc * (1.0 / (double)p->d);"),
    "gqa_map_modulo": ("int64_t kvh = h / (p->heads / p->kv_heads);", "int64_t kvh = h % p->kv_heads;"),
    "query_position_from_start": ("L.i = p->n - p->nq + r;", "L.i = r + (p->n - p->nq) / 2;"),
    "key_transposed": ("acc += qrow[t] * load_elem(k, p->dtype, base + t);",
                       "acc += qrow[t] * load_elem(k, p->dtype, kv_off + t * p->n + j) + 0.0 * base;"),
    "value_row_by_slot": ("int64_t base = kv_off + list[c] * p->d;", "int64_t base = kv_off + c * p->d;"),
    "no_normalisation": ("for (int64_t t = 0; t < p->d; ++t) o[t] /= l;", "(void)l;"),
    "bf16_widen_wrong": ("<< 16;", "<< 15;"),
    "anchor_dropped": ("w->member[0] = 1;", "w->member[0] = 0;"),
    "band_signed_halved": ("if (fabs(w->s[j]) > mabs) mabs = fabs(w->s[j]);",
                           "if (w->s[j] > mabs) mabs = w->s[j] * 0.5;"),
    "band_signed": ("if (fabs(w->s[j]) > mabs) mabs = fabs(w->s[j]);",
                    "if (w->s[j] > mabs) mabs = w->s[j];"),
    "k_minus_one": ("const int64_t kp = p->topk < n_r ? p->topk : n_r;",
                    "const int64_t kp = p->topk < n_r ? (p->topk > 0 ? p->topk - 1 : 0) : n_r;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new)
    csrc = tmp_path / "mutant.c"
    csrc.write_text(mutated)
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-fopenmp", "-fPIC", "-shared", "-w",
                           "-o", str(so), str(csrc), "-lm"])
    env = dict(os.environ, CONDENSATE_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"pins did not catch mutant {name}:\n{res.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_sweep_rejects_planted_mistake(name, tmp_path):
    """The property sweep (random shapes) alone also catches every planted mistake."""
    old, new = MUTANTS[name]
    src = open(SRC).read()
    csrc = tmp_path / "mutant.c"
    csrc.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-fopenmp", "-fPIC", "-shared", "-w",
                           "-o", str(so), str(csrc), "-lm"])
    env = dict(os.environ, CONDENSATE_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_sweep.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"the sweep did not catch mutant {name}:\n{res.stdout[-2000:]}"
