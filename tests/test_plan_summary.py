"""The opt-in plan summary (rpkv_plan_summary, RPKV_LOG_PLANS): host planning only."""
import os
import subprocess
import sys

import numpy as np
import pytest

import ragged_paged_kv_store_amd as rp
from tests import gpu_harness as H
from workloads import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_summary_counts_match_the_plan():
    spec = synth.full_config(5)
    plan = H.make_plan(spec)
    with pytest.raises(rp.RpkvError):
        plan.summary()                                  # nothing planned yet
    plan.plan_host(spec.cu_q, spec.L, spec.page_table.shape[1], None, spec.groups)
    info = plan.info()
    line = plan.summary()
    n = spec.n.astype(np.int64)
    ndec = int(((n > 0) & (n * spec.G <= 16)).sum())
    npre = int(((n > 0) & (n * spec.G > 16)).sum())
    assert line.startswith(f"batch {spec.bs} ({spec.T} tokens): {ndec} decode-type, {npre} prefill-type, 0 empty")
    assert f"{info['num_prefill_items']} MFMA tiles ({info['tiles_per_block']} per workgroup, " \
           f"{info['num_cascade_items']} in shared-prefix levels)" in line
    assert f"{info['num_decode_items']} split-KV chunks of {info['decode_chunk']} keys" in line
    assert f"{info['num_cascade_levels']} cascade levels (depth {info['cascade_depth']}" in line
    assert f"{info['num_partials']} partials, {info['num_merge_tokens']} tokens merged" in line
    assert f"metadata {info['metadata_bytes']} bytes" in line
    plan.close()


def test_summary_truncates_to_the_buffer():
    spec = synth.full_config(2)
    plan = H.make_plan(spec)
    plan.plan_host(spec.cu_q, spec.L, spec.page_table.shape[1], None, spec.groups)
    import ctypes
    buf = ctypes.create_string_buffer(b"x" * 24, 24)
    assert rp.lib.rpkv_plan_summary(plan._h, buf, 16) == 0
    assert len(buf.value) == 15 and buf.raw[15:16] == b"\0" and buf.raw[16:] == b"x" * 8
    plan.close()


@pytest.mark.parametrize("value,expect", [("1", True), ("0", False), (None, False)])
def test_log_plans_environment_switch(value, expect):
    env = dict(os.environ)
    env.pop("RPKV_LOG_PLANS", None)
    if value is not None:
        env["RPKV_LOG_PLANS"] = value
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from tests import gpu_harness as H\nfrom workloads import synth\n"
            "s = synth.full_config(3); p = H.make_plan(s)\n"
            "p.plan_host(s.cu_q, s.L, s.page_table.shape[1], None, s.groups)\n"
            "p.plan_host(s.cu_q, s.L, s.page_table.shape[1], None, s.groups)\n"
            "print(p.summary())\n") % ROOT
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    logged = [l for l in r.stderr.splitlines() if l.startswith("rpkv: ")]
    if expect:
        assert len(logged) == 2 and logged[1] == "rpkv: " + r.stdout.strip()
    else:
        assert not logged
