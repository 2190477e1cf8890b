"""The pins must catch plausible slips: plant each one in a scratch copy of
the oracle (on the CPU) and check that the pin suite then fails."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# the backward slips: one whole-branch autograd comparison catches each
BWD = "test_oracle_backward.py::test_branch_backward_matches_autograd[t16]"
E2E = "test_oracle_e2e.py::test_e2e_tiny_matches_brute_force"

MUTATIONS = [
    ("tie-break", "if (best < 0 || l[e] > l[best]) best = e;",
     "if (best < 0 || l[e] >= l[best]) best = e;", "test_oracle_pins.py"),
    ("gate/up swap", "h[f] = bf(to_bf(silu(a) * b));", "h[f] = bf(to_bf(silu(b) * a));",
     "test_oracle_pins.py"),
    ("wave index", "int32_t w = t / Tw;", "int32_t w = t % W;", "test_oracle_pins.py"),
    ("gates renormalised away", "gates[t * k + j] = (float)(exp((double)l[best] - m) / Z);",
     "gates[t * k + j] = (float)(exp((double)l[best] - m));", "test_oracle_pins.py"),
    ("latent weight transposed", "for (int32_t i = 0; i < D; ++i) acc += xr[i] * bf(w[i]);",
     "for (int32_t i = 0; i < D; ++i) acc += xr[i] * bf(w_ld_t[(int64_t)(i % L) * D + c]);",
     "test_oracle_pins.py"),
    ("shared expert dropped", "for (int32_t f = 0; f < Fs; ++f) o += h[sh * Fs + f] * bf(wd[f]);",
     "for (int32_t f = 0; f < Fs; ++f) o += (sh == 0) * h[sh * Fs + f] * bf(wd[f]);",
     "test_oracle_pins.py"),
    ("capacity off by one", "if (cap == 0 || pos < cap) {", "if (cap == 0 || pos <= cap) {",
     "test_oracle_pins.py"),
    ("receiver source order", "for (int32_t s = 0; s < R; ++s) {\n      int64_t a = ragged ? recv_offsets[s * W + w] : ((int64_t)s * W + w) * d->cap_send;\n      int64_t b = ragged ? recv_offsets[s * W + w + 1] : a + d->cap_send;\n      for (int64_t q = a * per; q < b * per; ++q) {\n        int32_t h = hdr[q];\n        if (h < 0",
     "for (int32_t s = R - 1; s >= 0; --s) {\n      int64_t a = ragged ? recv_offsets[s * W + w] : ((int64_t)s * W + w) * d->cap_send;\n      int64_t b = ragged ? recv_offsets[s * W + w + 1] : a + d->cap_send;\n      for (int64_t q = a * per; q < b * per; ++q) {\n        int32_t h = hdr[q];\n        if (h < 0",
     "test_oracle_pins.py"),
    ("fill not capped", "fill[p] = (cap == 0 || n[p] < cap) ? n[p] : cap;", "fill[p] = n[p];",
     "test_oracle_pins.py"),
    ("gate not applied", "for (int32_t c = 0; c < L; ++c) acc[c] += g * bf(returned[row * L + c]);",
     "for (int32_t c = 0; c < L; ++c) acc[c] += bf(returned[row * L + c]);", "test_oracle_pins.py"),
    ("down weight transposed", "acc += h[f] * bf(w[f]);",
     "acc += h[f] * bf(wd_t[(int64_t)f * L + (c % F)]);", "test_oracle_pins.py"),
    ("return segment order", "int32_t seg = dest_of(d, e) * W + w;",
     "int32_t seg = w * d->n_ranks + dest_of(d, e);", E2E + "[1.10/1.15]"),
    ("expert placement", "return e / (d->n_experts / d->n_ranks);", "return e % d->n_ranks;",
     "test_oracle_pins.py"),
    ("balance bias sign", "bias[i] = (float)(-alpha * (f - 1.0 / (double)E));",
     "bias[i] = (float)(alpha * (f - 1.0 / (double)E));", "test_oracle_balance.py"),
    ("bias subtracted", "for (int32_t e = 0; e < E; ++e) lb[e] = logits[t * E + e] + bias[e];",
     "for (int32_t e = 0; e < E; ++e) lb[e] = logits[t * E + e] - bias[e];",
     "test_oracle_balance.py"),
    ("expert 0 not counted", "if (topk[i] >= 0 && topk[i] < E) counts[topk[i]] += 1;",
     "if (topk[i] > 0 && topk[i] < E) counts[topk[i]] += 1;", "test_oracle_balance.py"),
    ("renormalised over k - 1",
     "      for (int32_t j = 0; j < k; ++j) z += exp((double)lb[topk[t * k + j]] - m);",
     "      for (int32_t j = 1; j < k; ++j) z += exp((double)lb[topk[t * k + j]] - m);",
     "test_oracle_balance.py"),
    ("window: last batch only",
     "    for (int32_t b = 0; b < n_batches; ++b) h += window[(int64_t)b * E + i];",
     "    for (int32_t b = n_batches - 1; b < n_batches; ++b) h += window[(int64_t)b * E + i];",
     "test_oracle_balance.py"),
    ("chunk demand: last chunk capped",
     "      demand[r * W + w] = (int32_t)(w + 1 < W ? fill[r * W + w] : left);",
     "      demand[r * W + w] = fill[r * W + w];", "test_oracle_pins.py"),
    ("chunk pool one chunk short",
     "  const int64_t cap = d->cap_send, pool = (int64_t)W * cap;",
     "  const int64_t cap = d->cap_send, pool = (int64_t)(W - 1) * cap;", "test_oracle_pins.py"),
    ("chunk rows offset by wave",
     "      if (d->wave_mode == 1) row = (int64_t)dest_of(d, e) * W * d->cap_send + s;",
     "      if (d->wave_mode == 1) row = (int64_t)(dest_of(d, e) * W + t / Tw) * d->cap_send + s;",
     "test_oracle_pins.py"),
    ("chunk combine row",
     "        row = (int64_t)dest_of(d, e) * W * d->cap_send + s; /* slot: position in the dest's pool */",
     "        row = (int64_t)seg * d->cap_send + s % d->cap_send;", E2E + "[chunks]"),
    ("dedup groups of three", "  if (c % 4 == 0) return 0;", "  if (c % 3 == 0) return 0;",
     "test_oracle_pins.py"),
    ("dedup row without its leader's id",
     "if (dest_of(d, tk[i]) == dest_of(d, e) && dedup_rank(d, tk, i) >= c) ids[m++] = tk[i];",
     "if (dest_of(d, tk[i]) == dest_of(d, e) && dedup_rank(d, tk, i) > c) ids[m++] = tk[i];",
     "test_oracle_pins.py"),
    ("dedup return slot ignored",
     "      if (d->dedup) row = row * 4 + dedup_rank(d, topk + t * k, j) % 4; /* return slot */",
     "      if (d->dedup) row = row * 4; /* return slot */", E2E + "[dedup_tight]"),
    ("silu derivative", "  return s * (1.0 + a * (1.0 - s));", "  return s;", BWD),
    ("shared d_b from b", "d_shared[(t * 2 * S + S + sh) * Fs + f] = to_bf(dh * silu(a));",
     "d_shared[(t * 2 * S + S + sh) * Fs + f] = to_bf(dh * b);", BWD),
    ("gate gradient sign", "      d_gates[t * k + j] = (float)dot;", "      d_gates[t * k + j] = (float)-dot;",
     BWD),
    ("expert d_u gate/up weights swapped",
     "acc += da[f] * bf(Wg[(int64_t)f * L + l]) + db[f] * bf(Wu[(int64_t)f * L + l]);",
     "acc += da[f] * bf(Wu[(int64_t)f * L + l]) + db[f] * bf(Wg[(int64_t)f * L + l]);",
     BWD),
    ("softmax normaliser term dropped", "      for (int32_t e = 0; e < E; ++e) dl[e] = -p[e] * s;",
     "      for (int32_t e = 0; e < E; ++e) dl[e] = 0.0;",
     "test_oracle_backward.py::test_route_backward_finite_differences"),
    ("return gradient not gated", "        d_returned[row * L + i] = to_bf(g * dyl[i]);",
     "        d_returned[row * L + i] = to_bf(dyl[i]);", BWD),
    ("dx without shared up path",
     "               bf(d_shared[(t * 2 * S + S + sh) * Fs + f]) * bf(ws_up[wi]);",
     "               0.0 * bf(ws_up[wi]);", BWD),
    ("expert down grad with u for h", "gd[j * WL + (int64_t)l * F + f] += dy[l] * h[f];",
     "gd[j * WL + (int64_t)l * F + f] += dy[l] * u[f % L];", BWD),
    ("ragged: no segment bound", "  if (s >= offsets[seg + 1] - offsets[seg]) return -1;\n",
     "", "test_oracle_backward.py::test_ragged_backward_bounds_and_sampled"),
    ("ragged bank groups read at fixed positions",
     "  return d->cap_send ? (int64_t)g * d->cap_recv : bank_offsets[g];",
     "  return (int64_t)g * d->cap_recv;",
     "test_oracle_backward.py::test_branch_backward_matches_autograd[t16_ragged_w1]"),
]


def _run_mutant(tmp_root, name, old, new, suite):
    """Exit status of the pin suite against a copy of the oracle with one slip
    planted (and the tail of its output)."""
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    if src.count(old) < 1:
        return None, f"mutation site for {name!r} not found"
    work = os.path.join(tmp_root, "m%d" % [m[0] for m in MUTATIONS].index(name))
    for d in ("oracle", "synth", "tests"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(work, d),
                        ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    with open(os.path.join(work, "oracle", "oracle.c"), "w") as f:
        f.write(src.replace(old, new, 1))
    p = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join("tests", suite)], cwd=work, capture_output=True,
                       text=True, timeout=600, env=_ONE_THREAD)
    return p.returncode, p.stdout[-2000:]


# children run side by side: one BLAS / OpenMP thread each
_ONE_THREAD = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1",
                   MKL_NUM_THREADS="1")


@pytest.fixture(scope="module")
def mutant_results(tmp_path_factory):
    """Every mutant's suite, run in parallel child processes (one CPU each)."""
    from concurrent.futures import ThreadPoolExecutor
    root = str(tmp_path_factory.mktemp("mutants"))
    workers = max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        futs = {m[0]: ex.submit(_run_mutant, root, *m) for m in MUTATIONS}
        return {k: f.result() for k, f in futs.items()}


@pytest.mark.parametrize("name,old,new,suite", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(mutant_results, name, old, new, suite):
    rc, out = mutant_results[name]
    assert rc is not None, out
    assert rc != 0, f"pins did not catch {name!r}:\n{out}"
