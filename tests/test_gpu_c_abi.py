"""The C ABI driven from plain C on the GPU: tests/c/run_from_c.c allocates
device memory with the HIP runtime, runs gla_chunk_fwd and one
gla_recurrent_step on a library pool, and writes the results; they must match
the fp64 oracle as the torch-driven tests do.  No torch touches the device in
that program."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import gen
import oracle
from gpu_util import assert_close

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bf16_raw(x):
    """Raw bf16 bits of float32 values that are exact in bf16."""
    return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_prefill_and_decode_from_c(tmp_path):
    import linear_attention_sequence_simple_amd as gla
    if shutil.which("gcc") is None or not os.path.exists(gla.lib_path()):
        pytest.skip("gcc or libgla.so missing")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    libdir = os.path.dirname(gla.lib_path())
    exe = str(tmp_path / "run_from_c")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "run_from_c.c"), "-o", exe,
                    "-L", libdir, "-lgla", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
                    "-Wl,-rpath," + libdir, "-Wl,-rpath," + os.path.join(rocm, "lib")], check=True)
    B, T, H = 2, 300, 2
    d = gen.make_inputs("fwd_bf16_b8_t2048", seed=31, B=B, T=T, H=H, S0="zero")
    for name in ("q", "k", "v"):
        _bf16_raw(d[name]).tofile(tmp_path / f"{name}.bf16")
    d["g"].astype(np.float32).tofile(tmp_path / "g.f32")
    x = gen.make_decode_step(B, 0, H=H, seed=31)
    for name in ("q", "k", "v"):
        _bf16_raw(x[name]).tofile(tmp_path / f"step_{name}.bf16")
    x["g"].astype(np.float32).tofile(tmp_path / "step_g.f32")
    S = gen.make_decode_state(B, H=H, seed=31)
    S.astype(np.float32).tofile(tmp_path / "pool.f32")
    print("case C ABI: prefill B=2 T=300 H=2, decode step on 2 slots", flush=True)
    r = subprocess.run([exe, str(tmp_path), str(B), str(T), str(H)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    o = np.fromfile(tmp_path / "o.f32", np.float32).reshape(B, T, H, 192)
    S_T = np.fromfile(tmp_path / "S_T.f32", np.float32).reshape(B, H, 96, 192)
    o_ref, S_ref = oracle.forward(d["q"], d["k"], d["v"], d["g"], None)
    assert_close(o.astype(np.float64), o_ref, 1e-2, "o (prefill from C)")
    assert_close(S_T.astype(np.float64), S_ref, 1e-2, "S_T (prefill from C)")
    so = np.fromfile(tmp_path / "step_o.f32", np.float32).reshape(B, H, 192)
    pool = np.fromfile(tmp_path / "pool_after.f32", np.float32).reshape(B, H, 96, 192)
    so_ref, pool_ref = oracle.step(S, x["q"], x["k"], x["v"], x["g"])
    assert_close(so.astype(np.float64), so_ref, 1e-4, "o (decode from C)")
    assert_close(pool.astype(np.float64), pool_ref, 1e-4, "pool (decode from C)")
