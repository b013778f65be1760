"""Plant plausible mistakes in copies of the CPU oracle and check that the
pins in tests/oracle_pins.py catch every one of them.

Each mutant is a textual edit of oracle.c (a dropped term, a wrong index or
divisor, a missing or misplaced rounding, a reordered reduction).  The copy is
built with gcc in a temporary directory and the whole pin suite runs against
it in a child process, so a mutant that reads out of bounds cannot take the
test runner down.  A mutant survives if every pin passes; none may.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "eps_dropped": ("sqrt(ss / (double)hidden + eps)", "sqrt(ss / (double)hidden)"),
    "eps_outside_root": ("1.0 / sqrt(ss / (double)hidden + eps)",
                         "1.0 / (sqrt(ss / (double)hidden) + eps)"),
    "mean_divisor_h_minus_1": ("ss / (double)hidden + eps", "ss / (double)(hidden - 1) + eps"),
    "mask_off_by_one": ("if (i < 0 || i >= num_rows)", "if (i < 0 || i > num_rows)"),
    "mask_negative_allowed": ("if (i < 0 || i >= num_rows)", "if (i >= num_rows)"),
    "slots_descending": ("for (int32_t k = 0; k < top_k; ++k) {\n        int64_t i = idx[k];",
                         "for (int32_t k = top_k - 1; k >= 0; --k) {\n        int64_t i = idx[k];"),
    "mul_then_add": ("acc[h] = fmaf(w, oracle_bf16_to_f32(row[h]), acc[h]);",
                     "acc[h] = w * oracle_bf16_to_f32(row[h]) + acc[h];"),
    "gain_center_dropped": ("g[h] = oracle_bf16_to_f32(norm_weight[h]) + gain_center;",
                            "g[h] = oracle_bf16_to_f32(norm_weight[h]);"),
    "gain_center_bf16": ("g[h] = oracle_bf16_to_f32(norm_weight[h]) + gain_center;",
                         "g[h] = oracle_bf16_to_f32(oracle_round_to_bf16("
                         "(double)(oracle_bf16_to_f32(norm_weight[h]) + gain_center)));"),
    "weight_applied_twice": ("if (!weight_before_norm)\n                y *= (double)g[h];",
                             "y *= (double)g[h];"),
    "weight_never_before": ("z[h] = weight_before_norm ? (double)acc[h] * (double)g[h] : (double)acc[h];",
                            "z[h] = (double)acc[h];"),
    "beam_first_rounding_skipped": ("float scaled = oracle_bf16_to_f32(r) * routed_scale;",
                                    "float scaled = acc[h] * routed_scale; (void)r;"),
    "beam_second_rounding_skipped": ("s[h] = (double)oracle_bf16_to_f32(sb[h]);",
                                     "s[h] = (double)scaled;"),
    "beam_post_weight_ignored": ("if (post_weight)\n                y *= (double)oracle_bf16_to_f32(post_weight[h]);",
                                 "(void)post_weight;"),
    "rne_ties_away": ("if (rem > 0.5 || (rem == 0.5 && fmod(lo, 2.0) != 0.0))", "if (rem >= 0.5)"),
    "rne_truncates": ("if (rem > 0.5 || (rem == 0.5 && fmod(lo, 2.0) != 0.0))", "if (0)"),
    "subnormal_grid": ("        ulp_exp = -133;", "        ulp_exp = -126;"),
    "token_major_transposed": ("token_rows + (int64_t)k * hidden", "token_rows + (int64_t)k"),
    "beam_token_stride": ("expert_outputs + t * top_k * (int64_t)hidden",
                          "expert_outputs + t * (int64_t)hidden"),
    "bf16_weight_as_integer": ("oracle_bf16_to_f32(w_bf16[k])", "(float)w_bf16[k]"),
    "weight_row_stride": ("(const float *)weights + t * top_k", "(const float *)weights + t"),
    "row_stride_ignored": ("rows + i * row_stride", "rows + i * (int64_t)hidden"),
    "output_sign": ("double y = z[h] * inv;", "double y = -z[h] * inv;"),
    "standalone_row_stride": ("const uint16_t *x = input + t * row_stride;",
                              "const uint16_t *x = input + t * (int64_t)hidden;"),
    "residual_dropped": ("(double)scale_x * v[h] +\n                         (double)scale_res * (double)oracle_bf16_to_f32(rr[h]);",
                         "(double)scale_x * v[h];"),
    "scales_swapped": ("(double)scale_x * v[h] +\n                         (double)scale_res *",
                       "(double)scale_res * v[h] +\n                         (double)scale_x *"),
    "next_norm_from_unrounded_hidden": ("v[h] = (double)oracle_bf16_to_f32(hr[h]);", "v[h] = sum;"),
    "next_weight_ignored": ("if (next_weight)\n                y *= (double)oracle_bf16_to_f32(next_weight[h]);",
                            "(void)next_weight;"),
    "residual_row_stride": ("rr = residual + t * (int64_t)hidden;", "rr = residual + t * row_stride;"),
    "consumer_post_norm_unrounded": ("v[h] = (double)oracle_bf16_to_f32(oracle_round_to_bf16(y));",
                                     "v[h] = y;"),
    "standalone_weight_first_ignored": ("z[h] = weight_before_norm ? v * (double)g[h] : v;",
                                        "z[h] = v;"),
}

_RUNNER = r"""
import importlib.util, sys, traceback
sys.path[:0] = [{root!r}, {tests!r}]
spec = importlib.util.spec_from_file_location("oracle_mutant", {init!r},
                                              submodule_search_locations=[{pkg!r}])
mod = importlib.util.module_from_spec(spec)
spec.loader.exec_module(mod)
import oracle_pins
failed = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(mod)
    except Exception as e:
        failed.append(pin.__name__)
print("FAILED:" + ",".join(failed))
sys.exit(1 if failed else 0)
"""


def _run_mutant(name, old, new, workdir):
    pkg = os.path.join(workdir, name)
    os.makedirs(pkg)
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), pkg)
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    n = src.count(old)
    assert n >= 1, f"mutant {name}: pattern not found in oracle.c"
    with open(os.path.join(pkg, "oracle.c"), "w") as f:
        f.write(src.replace(old, new))
    code = _RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"),
                          init=os.path.join(pkg, "__init__.py"), pkg=pkg)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=600, env=env)
    return name, p.returncode, (p.stdout + p.stderr)[-400:]


def test_every_mutant_is_caught():
    with tempfile.TemporaryDirectory() as d:
        workers = min(8, os.cpu_count() or 1)
        with cf.ThreadPoolExecutor(workers) as ex:
            results = list(ex.map(lambda kv: _run_mutant(kv[0], *kv[1], d), MUTANTS.items()))
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"


if __name__ == "__main__":
    with tempfile.TemporaryDirectory() as d:
        for name, (old, new) in MUTANTS.items():
            print(_run_mutant(name, old, new, d)[:2], flush=True)
