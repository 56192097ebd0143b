"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU,
in a temporary directory), builds it, and runs the pin suite against that copy in
a subprocess: the suite must fail.  The unmodified oracle passes the same suite
(tests/test_oracle_pins.py).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "rpkv_oracle.c")

MUTATIONS = {
    "mask_off_by_one": ("int64_t hi = a + 1 < pb->key_hi ? a + 1 : pb->key_hi;",
                        "int64_t hi = a < pb->key_hi ? a : pb->key_hi;"),
    "top_left_alignment": ("const int64_t a = L - n + r;", "const int64_t a = r;"),
    "gqa_modulo_map": ("kvh = h / G;", "kvh = h % Hkv;"),
    "slot_ignores_page_size": ("return page * page_size + pos % page_size;",
                               "return page + pos % page_size;"),
    "scale_dropped": ("x[j - lo] = pb->scale * dot;", "x[j - lo] = dot;"),
    "max_not_subtracted": ("double w = exp(x[j - lo] - m);", "double w = exp(x[j - lo]);"),
    "lse_sign": ("*lse = m + log(Z);", "*lse = m - log(Z);"),
    "not_normalised": ("for (int32_t d = 0; d < D; ++d) out[d] /= Z;", ""),
    "v_from_k_pool": ("out[d] += w * up(pb->vpool, vbase + d, pb->dtype);",
                      "out[d] += w * up(pb->kpool, vbase + d, pb->dtype);"),
    "query_row_uses_kv_head": ("const int64_t qbase = ((int64_t)t * Hq + h) * D;",
                               "const int64_t qbase = ((int64_t)t * Hq + kvh) * D;"),
    "merge_weight_sign": ("double w = exp(l - M);", "double w = exp(M - l);"),
    "store_swaps_k_and_v": (
        "memcpy((char *)kpool + s * row_bytes, (const char *)k + t * row_bytes, (size_t)row_bytes);",
        "memcpy((char *)kpool + s * row_bytes, (const char *)v + t * row_bytes, (size_t)row_bytes);"),
    "last_index_off_by_one": ("out[i] = (cu_q[i + 1] > cu_q[i]) ? cu_q[i + 1] - 1 : -1;",
                              "out[i] = (cu_q[i + 1] > cu_q[i]) ? cu_q[i + 1] : -1;"),
    "position_off_by_one": ("int32_t pos = num_computed[i] + r;",
                            "int32_t pos = num_computed[i] + r + 1;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_fail_on_planted_mistake(name, tmp_path):
    orig, repl = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(orig) == 1, f"mutation anchor not unique/present: {name}"
    mutated = src.replace(orig, repl)
    c = tmp_path / "mut.c"
    so = tmp_path / "libmut.so"
    c.write_text(mutated)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-o", str(so), str(c),
                           "-lm", "-lpthread"])
    env = dict(os.environ, RPKV_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutation {name}:\n{r.stdout[-2000:]}"


# ---------------------------------------------------------------- prefix tree
TREE_SRC = os.path.join(ROOT, "oracle", "prefix_tree.py")
TREE_MUTATIONS = {
    "offer_rounds_up": ("return (int(L) - int(n)) // int(P)",
                        "return -(-(int(L) - int(n)) // int(P))"),
    "offer_counts_new_tokens": ("return (int(L) - int(n)) // int(P)", "return int(L) // int(P)"),
    "shallowest_depth": ("depth_of[s] = max(depth_of.get(s, 0), k)",
                         "depth_of[s] = depth_of.get(s, k)"),
    "singleton_nodes": ("if len(members) >= 2:", "if len(members) >= 1:"),
    "prune_from_root": ("base = 0 if a is None else depth_of[a] * P", "base = 0"),
    "largest_parent": ("(best is None or len(t) < len(best))",
                       "(best is None or len(t) > len(best))"),
    "ineligible_join": ("E = [j for j in range(bs) if eligible[j]]", "E = list(range(bs))"),
}

_TREE_RUNNER = """
import importlib.util, sys
spec = importlib.util.spec_from_file_location("oracle.prefix_tree", sys.argv[1])
mod = importlib.util.module_from_spec(spec)
sys.modules["oracle.prefix_tree"] = mod
spec.loader.exec_module(mod)
import oracle
oracle.prefix_tree = mod
import pytest
sys.exit(pytest.main(["-x", "-q", "-p", "no:cacheprovider", sys.argv[2]]))
"""


@pytest.mark.parametrize("name", sorted(TREE_MUTATIONS))
def test_tree_pins_fail_on_planted_mistake(name, tmp_path):
    orig, repl = TREE_MUTATIONS[name]
    src = open(TREE_SRC).read()
    assert src.count(orig) == 1, f"mutation anchor not unique/present: {name}"
    mod = tmp_path / "prefix_tree_mut.py"
    mod.write_text(src.replace(orig, repl))
    r = subprocess.run([sys.executable, "-c", _TREE_RUNNER, str(mod),
                        os.path.join(ROOT, "tests", "test_oracle_prefix_tree.py")],
                       cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutation {name}:\n{r.stdout[-2000:]}"


def test_tree_runner_passes_unmodified(tmp_path):
    mod = tmp_path / "prefix_tree_copy.py"
    mod.write_text(open(TREE_SRC).read())
    r = subprocess.run([sys.executable, "-c", _TREE_RUNNER, str(mod),
                        os.path.join(ROOT, "tests", "test_oracle_prefix_tree.py")],
                       cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
