"""Plants one plausible mistake at a time in a copy of the oracle (on the CPU)
and checks that the pin suite rejects every such copy.  A mistake the pins
could not see would make them worthless as evidence for the oracle."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_predicate.py", "tests/test_oracle_method.py",
        "tests/test_oracle_codecs.py"]

# (name, original text, planted mistake)
MUTANTS = [
    ("residual_dropped", "if (residual) s = s + (float)", "if (0) s = s + (float)"),
    ("round_reduced_ignored", "if (round_reduced) s = (float)oracle_round(f, (double)s);", ""),
    ("sum_in_fp64", "float s = (float)oracle_decode(f, partials[0][row + h]);",
     "double s = oracle_decode(f, partials[0][row + h]);"),
    ("gemma_sign", "gemma ? 1.0 + w : w", "gemma ? 1.0 - w : w"),
    ("gemma_ignored", "gemma ? 1.0 + w : w", "w"),
    ("mean_over_h_minus_1", "ss / (double)H", "ss / (double)(H - 1)"),
    ("eps_dropped", "sqrt(ss / (double)H + (double)eps)", "sqrt(ss / (double)H)"),
    ("weight_dropped", "(double)acc[h] * rstd * w_eff", "(double)acc[h] * rstd"),
    ("last_partial_skipped", "for (int r = 1; r < W; ++r)", "for (int r = 1; r < W - 1; ++r)"),
    ("ties_away_from_zero", "frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) == 1.0)",
     "frac >= 0.5"),
    ("subnormal_quantum", "v = ldexp((double)m, F.emin - F.mant_bits);",
     "v = ldexp((double)m, F.emin - F.mant_bits - 1);"),
    ("fp8_no_saturation", "v = F.has_inf ? INFINITY : F.maxval;", "v = INFINITY;"),
    ("fp8_fnuz_scale", "amax / 448.0", "amax / 240.0"),
    ("group_amax_first_group", "fabs(row_exact[g * group + j])", "fabs(row_exact[j])"),
    ("qk_weight_shard_offset", "oracle_decode(f, q_w[r * q_size + j])",
     "oracle_decode(f, q_w[j])"),
    ("qk_mean_per_shard", "ssq / (double)(W * q_size)", "ssq / (double)q_size"),
    ("qk_k_uses_q_scale", "y = oracle_decode(f, x[q_size + j]) * rk *",
     "y = oracle_decode(f, x[q_size + j]) * rq *"),
    ("tokens_from_first_dim", "if (numel / hidden > 80) return 0;",
     "if (numel / hidden > 81) return 0;"),
    ("byte_cap_inclusive", "return total_bytes < 256 * 1024;",
     "return total_bytes <= 256 * 1024;"),
    ("pack_limit", "hidden / pack > 1024", "hidden / pack > 1025"),
    ("w2_after_topology", "if (W == 2) return 1;\n    if (!fully_connected) return 0;",
     "if (!fully_connected) return 0;\n    if (W == 2) return 1;"),
]


def _run_mutant(workdir, name, orig, bad):
    src = open(oracle.SRC).read()
    if src.count(orig) < 1:
        return name, None, f"mutation site of {name} not found in oracle.c"
    d = os.path.join(workdir, name)
    os.makedirs(d, exist_ok=True)
    mutant_c = os.path.join(d, "oracle_mutant.c")
    with open(mutant_c, "w") as f:
        f.write(src.replace(orig, bad))
    lib = oracle.compile_c(mutant_c, os.path.join(d, "liboracle_mutant.so"))
    env = dict(os.environ, ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PINS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def mutant_results(tmp_path_factory):
    """Runs the pin suite against every planted mistake, several at a time."""
    workdir = str(tmp_path_factory.mktemp("mutants"))
    workers = min(8, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        futs = [ex.submit(_run_mutant, workdir, *m) for m in MUTANTS]
        return {f.result()[0]: f.result()[1:] for f in futs}


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_pins_reject_planted_mistake(mutant_results, name):
    rc, out = mutant_results[name]
    assert rc == 1, f"{name}: the pins did not fail (rc={rc})\n{out}"
