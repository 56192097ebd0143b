"""The C ABI from plain C: tests/c/abi_host.c is compiled with gcc as C11 against
include/rpkv.h, linked to the built library and run (host-only calls, no GPU);
its report must agree with the planner's documented behaviour."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "ragged_paged_kv_store_amd", "_build")


@pytest.fixture(scope="module")
def report(tmp_path_factory):
    if not os.path.exists(os.path.join(LIB_DIR, "librpkv.so")):
        pytest.skip("library not built")
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    exe = str(tmp_path_factory.mktemp("cabi") / "abi_host")
    subprocess.check_call(["gcc", "-std=c11", "-Wall", "-Werror", "-pedantic",
                           "-I", os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "tests", "c", "abi_host.c"),
                           "-L", LIB_DIR, "-lrpkv", "-Wl,-rpath," + LIB_DIR, "-o", exe])
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    return dict(line.split(" ", 1) for line in out.stdout.strip().splitlines() if " " in line)


def test_header_is_plain_c_and_host_calls_work(report):
    assert report["supports"] == "0"
    assert report["supports_bad"].startswith("2 ")      # UNSUPPORTED
    assert report["plan"] == "0"
    assert report["tokens"] == "342"
    assert report["max_seqlen_k"] == "1000"
    # 32 heads over 8 KV heads: G = 4, tiles of 32 tokens: ceil(300/32) + ceil(40/32)
    assert int(report["prefill_items"]) >= (10 + 2) * 8
    assert int(report["decode_items"]) >= 2 * 8          # two decodes, 8 KV heads
    assert report["last"] == "299 339 340 341"
    assert int(report["decode_list"]) == int(report["decode_items"])
    assert report["tiles_per_block"] == "1"              # short tiles: one per workgroup
    tpb, npre, pad = report["pairs"].split()
    assert tpb == "2" and npre == report["prefill_items"] and pad == "0"
    assert report["tpb_bad"] == "1"                      # INVALID_ARG
    assert report["plan_bad"] == "1 msg"                 # INVALID_ARG with a message


@pytest.mark.gpu
def test_c_program_forward_matches_oracle(tmp_path):
    """tests/c/abi_forward.c (plain C, HIP runtime API for device memory) runs one
    step of the reduced Llama-3-8B mixed batch through rpkv_prepare_metadata and
    rpkv_forward; its output is within the bf16 bar of the fp64 oracle and its
    K pool is bit-exact after the store."""
    import numpy as np
    import torch

    import oracle
    from workloads import synth
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = str(tmp_path / "abi_forward")
    subprocess.check_call(["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "tests", "c", "abi_forward.c"),
                           "-L", LIB_DIR, "-lrpkv", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
                           "-lm", "-Wl,-rpath," + LIB_DIR, "-o", exe])
    spec = synth.small_config(2)
    ht = synth.host_tensors(spec)
    ref, _, kp_ref, _ = oracle.store_then_attend(spec, ht, nthreads=8)
    d = tmp_path
    cols = spec.page_table.shape[1]
    np.array([spec.Hq, spec.Hkv, spec.D, spec.P, spec.num_pages, spec.bs, spec.T, cols],
             np.int32).tofile(d / "meta.bin")
    spec.cu_q.astype(np.int32).tofile(d / "cu.bin")
    spec.L.astype(np.int32).tofile(d / "L.bin")
    np.ascontiguousarray(spec.page_table, np.int32).tofile(d / "pt.bin")
    spec.slot_mapping.astype(np.int32).tofile(d / "sm.bin")
    for name in ("q", "k", "v", "kpool", "vpool"):
        np.ascontiguousarray(getattr(ht, name)).tofile(d / f"{name}.bin")
    r = subprocess.run([exe, str(d)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    out = np.fromfile(d / "out.bin", np.uint16).reshape(spec.T, spec.Hq, spec.D)
    got = synth.bf16_bits_to_f32(out).astype(np.float64)
    err = float(np.abs(got - ref).max())
    assert err <= 2e-2, f"max abs err {err:.3e}"
    kp = np.fromfile(d / "kpool_after.bin", np.uint16).reshape(kp_ref.shape)
    assert np.array_equal(kp, kp_ref)
