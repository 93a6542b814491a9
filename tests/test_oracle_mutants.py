"""Planted mistakes in the oracle, on the CPU: each entry below alters one
step of oracle/santa_oracle.c the way a plausible slip would (a dropped
term, a wrong sign, an index off by one or taken from the wrong axis, a
transposed operand, a tie rule turned around), builds that copy, and runs
the oracle's pins (tests/test_oracle.py) against it.  Every altered copy
must fail at least one pin: otherwise the pins could not tell that mistake
from the method.  The oracle built in place is never touched.

A change that cannot alter any result is not listed: for instance, dropping
the inverse CDF's guard against selecting a zero-mass last token, which no
threshold in [0, 1) reaches, since the total is summed in the order of the
prefix and the last token with mass closes its cell at exactly 1."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "santa_oracle.c")

# (name, text in santa_oracle.c, replacement, number of occurrences replaced)
MUTANTS = [
    # scores and the softmax
    ("scores without the scale", "x[j] = (double)p->scale * dot;", "x[j] = dot;", 1),
    ("GQA head map modulo instead of division",
     "return h / (p->num_q_heads / p->num_kv_heads);", "return h % p->num_kv_heads;", 1),
    ("softmax exponent with the sign flipped", "e[j] = exp(x[j] - m);", "e[j] = exp(m - x[j]);", 1),
    ("exact decode without the 1/Z", "double a = e[j] / Z;", "double a = e[j];", 1),
    ("exact decode drops the last key", "for (int j = 0; j < n; ++j) {\n            double a = e[j] / Z;",
     "for (int j = 0; j < n - 1; ++j) {\n            double a = e[j] / Z;", 1),
    ("scores drop the last feature", "for (int i = 0; i < d; ++i)\n            dot += load_val(q, qoff + i",
     "for (int i = 0; i < d - 1; ++i)\n            dot += load_val(q, qoff + i", 1),
    ("exact decode sums K rows instead of V rows",
     "for (int i = 0; i < d; ++i) o[i] += a * load_val(v, off + i, p->kv_fmt);",
     "for (int i = 0; i < d; ++i) o[i] += a * load_val(k, off + i, p->kv_fmt);", 1),
    # storage formats and layouts
    ("e4m3 exponent bias 8", "ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)", 1),
    ("e4m3 subnormal scale 2^-7", "ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)", 1),
    ("contiguous KV with batch and head swapped",
     "return (((size_t)b * p->num_kv_heads + g) * p->max_seq_len + j) * d;",
     "return (((size_t)g * p->batch + b) * p->max_seq_len + j) * d;", 1),
    ("paged KV rows reversed within a page",
     "* p->page_size + j % p->page_size) * d;", "* p->page_size + (p->page_size - 1 - j % p->page_size)) * d;", 1),
    # inverse CDF and the threshold generators
    ("inverse CDF with right-closed cells", "while (j < n && !(F[j] > t[m])) ++j;",
     "while (j < n && !(F[j] >= t[m])) ++j;", 1),
    ("systematic offset taken as a [0,1) uniform", "t[m] = U + (double)m / (double)S;",
     "t[m] = (U + (double)m) / (double)S;", 1),
    ("stratified uniforms in reverse stratum order", "t[m] = ((double)m + u01[m]) / (double)S;",
     "t[m] = ((double)m + u01[S - 1 - m]) / (double)S;", 1),
    ("i.i.d. thresholds left unsorted", "qsort(t, (size_t)S, sizeof(double), cmp_double);", "", 1),
    ("CDF cell of a token closed at the next token's edge", "        hi[m] = F[j];",
     "        hi[m] = (j + 1 < n) ? F[j + 1] : 1.0;", 1),
    # estimators and their exact moments
    ("repeated indices counted once",
     "        size_t off = kv_row_offset(p, b, g, idx[m]);\n        for (int i = 0; i < d; ++i) out[i] += load_val(v, off + i, p->kv_fmt);",
     "        if (m > 0 && idx[m] == idx[m - 1]) continue;\n        size_t off = kv_row_offset(p, b, g, idx[m]);\n"
     "        for (int i = 0; i < d; ++i) out[i] += load_val(v, off + i, p->kv_fmt);", 1),
    ("tile counts indexed by threshold instead of token", "tc[J[m] / p->tile_len] += 1;",
     "tc[m * mnt / S] += 1;", 1),
    ("flash offset not scaled to the tile budget", "uf = U * (double)nt;", "uf = U;", 1),
    ("flash tile weights with the exponent sign flipped", "zt[tt] * exp(mt[tt] - M)", "zt[tt] * exp(M - mt[tt])", 2),
    ("flash indices left tile-local", "for (int m = 0; m < Sf; ++m) J[m] += j0;", "", 1),
    ("flash replay ignores the tile weights", "for (int i = 0; i < d; ++i) o[i] += pt * ot[i];",
     "for (int i = 0; i < d; ++i) o[i] += ot[i] / ntile;", 1),
    ("systematic moments weigh intervals by length, not length * S", "double prob = (c - a) * (double)S;",
     "double prob = (c - a);", 1),
    ("systematic moments miss the last breakpoint",
     "for (int j = 0; j < n - 1; ++j) {\n        run += w[j];\n        double F = run / z;",
     "for (int j = 0; j < n - 2; ++j) {\n        run += w[j];\n        double F = run / z;", 1),
    ("flash moments weigh tiles by their unnormalised mass", "est[i] += (zt / Z) * ot[i];",
     "est[i] += zt * ot[i];", 1),
    ("variance without the squared mean", "*var_trace = second - mm;", "*var_trace = second;", 2),
    # Bernoulli scores
    ("Bernoulli keep decision not strict", "if (prod < mag) kept += 1;", "if (prod <= mag) kept += 1;", 1),
    ("Bernoulli coefficients lose the sign", "c[i] = sgn * kept;", "c[i] = kept;", 1),
    ("Bernoulli score without 1/draws", "double coef = (double)p->scale * ((double)a / (double)draws);",
     "double coef = (double)p->scale * (double)a;", 1),
    ("Bernoulli uniforms read transposed", "float ur = u[(size_t)r * d + i];",
     "float ur = u[(size_t)i * draws + r];", 1),
    ("mean group query left as the sum", "qf[i] = s * (1.0f / (float)G);", "qf[i] = s;", 1),
    ("mean group query draws per q head",
     "size_t owner = group_mean ? (size_t)b * p->num_kv_heads + kv_head_of(p, h)",
     "size_t owner = group_mean ? (size_t)b * p->num_kv_heads + h % p->num_kv_heads", 1),
]


def _patched_source(old, new, count):
    src = open(SRC).read()
    assert src.count(old) == count, (old, src.count(old))
    return src.replace(old, new)


def test_mutants_apply_to_the_current_source():
    for name, old, new, count in MUTANTS:
        assert _patched_source(old, new, count) != open(SRC).read(), name


def _run(tmp, i, name, old, new, count):
    from oracle import build as obuild
    src = os.path.join(tmp, f"mutant{i}.c")
    lib = os.path.join(tmp, f"libmutant{i}.so")
    with open(src, "w") as f:
        f.write(_patched_source(old, new, count))
    obuild.build(src=src, out=lib)
    env = dict(os.environ, ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"),
                        "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-400:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    workers = max(1, min(6, (os.cpu_count() or 2) - 1))
    with ThreadPoolExecutor(workers) as ex:
        res = list(ex.map(lambda a: _run(str(tmp_path), *a), [(i, *m) for i, m in enumerate(MUTANTS)]))
    survivors = [(name, out) for name, rc, out in res if rc == 0]
    errors = [(name, rc, out) for name, rc, out in res if rc not in (0, 1)]
    assert not errors, errors          # 1 = some pin failed; anything else is a broken run
    assert not survivors, [n for n, _ in survivors]
