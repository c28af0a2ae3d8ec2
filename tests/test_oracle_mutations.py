"""The oracle's pins must catch plausible mistakes. Each case plants one
mistake in a copy of oracle/moe_oracle.c (on the CPU: a temporary build that
nothing else loads), runs the pin tests of that stage against it and expects
them to fail. A mistake that the pins let through would mean a bug of that
kind in the oracle could hide."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

ROUTER = "tests/test_oracle_router.py"
INDICES = "tests/test_oracle_indices.py"
FINALIZE = "tests/test_oracle_finalize.py"
DTYPES = "tests/test_oracle_dtypes.py"
SCOREFN = "tests/test_oracle_scorefn.py"

MUTATIONS = [
    ("bias left out of the selection", ROUTER,
     "b[e] = s[e] + load_as_f32(bias, bias_dtype, e);", "b[e] = s[e];"),
    ("bias added into the weights", ROUTER,
     "double w = (double)s[e];", "double w = (double)b[e];"),
    ("group score is the maximum only", ROUTER,
     "score = grp[0].v + grp[1].v;", "score = grp[0].v;"),
    ("group score adds the wrong second term", ROUTER,
     "score = grp[0].v + grp[1].v;", "score = grp[0].v + grp[S - 1].v;"),
    ("ties broken towards the higher index", ROUTER,
     "if (x->id < y->id) return -1;\n    if (x->id > y->id) return 1;",
     "if (x->id > y->id) return -1;\n    if (x->id < y->id) return 1;"),
    ("one group too few kept", ROUTER,
     "for (int32_t r = 0; r < topk_group; ++r)", "for (int32_t r = 0; r + 1 < topk_group; ++r)"),
    ("group restriction ignored", ROUTER, "if (kept[e / S]) {", "if (1) {"),
    ("expert-to-group map transposed", ROUTER, "if (kept[e / S]) {", "if (kept[e % n_groups]) {"),
    ("normalisation skipped", ROUTER, "if (norm_weights) w = w / sum;", ";"),
    ("scaling factor skipped", ROUTER, "w = w * (double)routed_scaling_factor;", ";"),
    ("normaliser drops the last weight", ROUTER,
     "for (int32_t k = 0; k < K; ++k) sum += (double)s[cand[k].id];",
     "for (int32_t k = 0; k + 1 < K; ++k) sum += (double)s[cand[k].id];"),
    ("bucket sort not stable", INDICES,
     "for (int64_t i = 0; i < N; ++i) {\n        const int32_t e = topk_ids[i];",
     "for (int64_t i = N - 1; i >= 0; --i) {\n        const int32_t e = topk_ids[i];"),
    ("CSR tail not N", INDICES,
     "expert_start_indices[j] = (uint32_t)N;", "expert_start_indices[j] = 0;"),
    ("expert id tail not -1", INDICES, "expert_ids[j] = -1;", "expert_ids[j] = 0;"),
    ("usage stats swapped", INDICES,
     "expert_usage_stats[0] = largest;\n    expert_usage_stats[1] = active;",
     "expert_usage_stats[1] = largest;\n    expert_usage_stats[0] = active;"),
    ("restore off by one", INDICES,
     "restore_token_order[i] = p;", "restore_token_order[i] = p + 1 < (uint32_t)N ? p + 1 : p;"),
    ("order holds the token, not the slot", INDICES,
     "token_expert_order[p] = (uint32_t)i;", "token_expert_order[p] = (uint32_t)(i / 2);"),
    ("inactive experts listed", INDICES,
     "if (count[e] > 0) {\n            expert_ids[active] = e;",
     "if (count[e] >= 0) {\n            expert_ids[active] = e;"),
    ("scale offsets not padded", INDICES,
     "offset += (count[e] + align - 1) / align * align;", "offset += count[e];"),
    ("scale offsets rounded down", INDICES,
     "offset += (count[e] + align - 1) / align * align;", "offset += count[e] / align * align;"),
    ("accumulator wider than fp32", FINALIZE,
     ["float* acc = (float*)malloc(sizeof(float)",
      "acc[h] = fmaf(w, load_as_f32(down, down_dtype, row * H + h), acc[h]);"],
     ["double* acc = (double*)malloc(sizeof(double)",
      "acc[h] = fma((double)w, (double)load_as_f32(down, down_dtype, row * H + h), acc[h]);"]),
    ("multiply then add instead of a fused multiply-add", FINALIZE,
     "acc[h] = fmaf(w, load_as_f32(down, down_dtype, row * H + h), acc[h]);",
     "{ float p_ = w * load_as_f32(down, down_dtype, row * H + h); acc[h] = acc[h] + p_; }"),
    ("k summed in reverse", FINALIZE,
     "for (int32_t k = 0; k < K; ++k) {\n                    const int64_t row",
     "for (int32_t k = K - 1; k >= 0; --k) {\n                    const int64_t row"),
    ("weight index transposed", FINALIZE,
     "load_as_f32(router_weight, weight_dtype, t * K + k)",
     "load_as_f32(router_weight, weight_dtype, (k * T + t) % (T * K))"),
    ("restore read as its inverse", FINALIZE,
     "const int64_t row = (int64_t)restore_order[t * K + k];",
     "int64_t row = 0;\n                    for (int64_t q = 0; q < N; ++q) if (restore_order[q] == (uint32_t)(t * K + k)) row = q;"),
    ("bf16 conversion truncates", FINALIZE, "u += 0x7fffu + lsb;", "(void)lsb;"),
    ("bf16 ties rounded away from zero", FINALIZE, "u += 0x7fffu + lsb;", "u += 0x8000u; (void)lsb;"),
    ("binary16 rounding truncates", DTYPES,
     "const uint32_t rounded = a + 0x0fffu + ((a >> 13) & 1u);", "const uint32_t rounded = a;"),
    ("binary16 ties rounded away from zero", DTYPES,
     "a + 0x0fffu + ((a >> 13) & 1u)", "a + 0x1000u"),
    ("binary16 subnormals truncated", DTYPES, "(uint16_t)nearbyintf(scaled)", "(uint16_t)scaled"),
    ("binary16 overflow threshold too low", DTYPES, "if (a >= 0x477ff000u)",
     "if (a >= 0x477fe000u)"),
    ("binary16 exponent rebias off by one", DTYPES, "((ex + 112u) << 23)", "((ex + 111u) << 23)"),
    ("binary16 output through bf16 rounding", DTYPES,
     "((uint16_t*)p)[i] = moe_oracle_f32_to_f16(v);", "((uint16_t*)p)[i] = moe_oracle_f32_to_bf16(v);"),
    ("bias read in the scores' dtype", DTYPES,
     "b[e] = s[e] + load_as_f32(bias, bias_dtype, e);",
     "b[e] = s[e] + load_as_f32(bias, scores_dtype, e);"),
    ("sigmoid of the negated logit", SCOREFN, "exp(-(double)s[e])", "exp((double)s[e])"),
    ("softmax sum misses the last expert", SCOREFN,
     "const double sum = moe_oracle_pairwise_sum(ex, E);",
     "const double sum = moe_oracle_pairwise_sum(ex, E - 1);"),
    ("softmax evaluated in binary32", SCOREFN,
     "s[e] = (float)(ex[e] / sum);", "s[e] = expf(s[e] - (float)m) / (float)sum;"),
    ("softmax denominator summed left to right", SCOREFN,
     "const double sum = moe_oracle_pairwise_sum(ex, E);",
     "double sum = 0.0;\n        for (int32_t e = 0; e < E; ++e) sum += ex[e];"),
    ("pairwise sum taken left to right", SCOREFN,
     "for (int64_t w = 1; w < P; w *= 2)\n        for (int64_t i = 0; i < P; i += 2 * w) t[i] = t[i] + t[i + w];",
     "for (int64_t i = 1; i < P; ++i) t[0] = t[0] + t[i];"),
    ("exp series one term short", SCOREFN,
     ["for (int n = 2; n <= 13; ++n)", "for (int n = 12; n >= 0; --n)"],
     ["for (int n = 2; n <= 12; ++n)", "for (int n = 11; n >= 0; --n)"]),
    ("exp reduction without the low part of ln 2", SCOREFN, "r = fma(-kd, LN2_LO, r);", ";"),
    ("exp scaled by 2^(k+1)", SCOREFN, "const int k1 = k / 2, k2 = k - k1;",
     "const int k1 = k / 2, k2 = k - k1 + 1;"),
]


def _run_mutant(mutation, workdir):
    """Build the oracle with one planted mistake and run the pins of its
    stage against that build (in a child process). Returns (returncode,
    tail of its output)."""
    name, tests, old, new = mutation
    src = open(SRC).read()
    olds, news = (old, new) if isinstance(old, list) else ([old], [new])
    for o, n in zip(olds, news):
        if src.count(o) < 1:
            return None, "mutation no longer applies: " + name
        src = src.replace(o, n)
    d = os.path.join(workdir, "m%d" % MUTATIONS.index(mutation))
    os.makedirs(d, exist_ok=True)
    mutated = os.path.join(d, "moe_oracle_mutant.c")
    with open(mutated, "w") as f:
        f.write(src)
    lib = os.path.join(d, "libmoe_oracle_mutant.so")
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                    "-o", lib, mutated, "-lm"], check=True, capture_output=True)
    # one OpenMP thread per child: several children run side by side
    env = dict(os.environ, MOE_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", tests], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def mutant_results(tmp_path_factory):
    """Results of every mutant, computed once, a few children at a time
    (each child is dominated by its interpreter start-up). Under pytest-xdist
    each case runs its own mutant instead."""
    if os.environ.get("PYTEST_XDIST_WORKER"):
        return None
    workdir = str(tmp_path_factory.mktemp("mutants"))
    workers = max(1, min(4, (os.cpu_count() or 1) // 2))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda m: _run_mutant(m, workdir), MUTATIONS))
    return {m[0]: r for m, r in zip(MUTATIONS, results)}


@pytest.mark.parametrize("mutation", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(mutation, mutant_results, tmp_path):
    name = mutation[0]
    if mutant_results is None:
        rc, out = _run_mutant(mutation, str(tmp_path))
    else:
        rc, out = mutant_results[name]
    assert rc is not None, out
    assert rc != 0, "pins did not catch: %s\n%s" % (name, out)
