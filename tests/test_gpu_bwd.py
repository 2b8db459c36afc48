"""Backward parity: gla_chunk_bwd on the GPU against the fp64 oracle backward."""
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, assert_close_bf16_out, inputs, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL = 1e-2


def run_bwd(d, S0=True, dS_T=True, out_dtype=torch.float32, segments=None):
    import linear_attention_sequence_simple_amd as gla
    old = os.environ.get("GLA_BWD_SEGMENTS")
    if segments is not None:
        os.environ["GLA_BWD_SEGMENTS"] = str(segments)
    try:
        r = gla.gla_chunk_bwd(to_dev(d["q"], torch.bfloat16), to_dev(d["k"], torch.bfloat16),
                              to_dev(d["v"], torch.bfloat16), to_dev(d["g"], torch.float32),
                              to_dev(d["dO"], torch.bfloat16),
                              S0=to_dev(d["S0"], torch.float32) if S0 else None,
                              dS_T=to_dev(d.get("dS_T"), torch.float32) if dS_T else None,
                              out_dtype=out_dtype, want_dS0=True)
        torch.cuda.synchronize()
    finally:
        if segments is not None:
            if old is None:
                os.environ.pop("GLA_BWD_SEGMENTS")
            else:
                os.environ["GLA_BWD_SEGMENTS"] = old
    return [to_np(x) for x in r]


def check(d, got, S0=True, dS_T=True):
    ref = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["dO"], d["S0"] if S0 else None,
                          d.get("dS_T") if dS_T else None)
    for name, x, y in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        assert_close(x, y, TOL, name)
    dg, dg_ref = got[3], ref[3]
    if np.all(dg_ref == 0):
        # no decay gradient at all (gamma == 0): compare with the scale of the
        # terms that cancel, q.dq
        scale = np.sqrt(np.mean(np.einsum("bthd,bthd->bth", d["q"], ref[0]) ** 2))
        assert np.max(np.abs(dg)) <= TOL * scale
    else:
        assert_close(dg, dg_ref, TOL, "dg")
    if S0 or dS_T:
        assert_close(got[4], ref[4], TOL, "dS0")


@pytest.mark.parametrize("T", [1, 77, 128, 200, 300, 513])
@pytest.mark.parametrize("s0,dst", [(True, True), (False, False)])
def test_reduced(T, s0, dst):
    d = inputs("bwd_bf16_b4_t4096", seed=T, B=2, T=T, H=2, S0="normal0.1", with_dO=True, with_dS_T=True)
    print(f"case bwd T={T} S0={s0} dS_T={dst}", flush=True)
    got = run_bwd(d, s0, dst)
    check(d, got, s0, dst)


@pytest.mark.parametrize("B,T,H", [(128, 3, 16), (64, 130, 2)])
def test_wide_batches(B, T, H):
    """Many short sequences (2,048 (b, h) pairs for B=128, H=16): every
    gradient against the oracle."""
    d = inputs("bwd_bf16_b4_t4096", seed=5, B=B, T=T, H=H, S0="normal0.1", with_dO=True, with_dS_T=True)
    print(f"case bwd wide batch B={B} T={T} H={H}", flush=True)
    check(d, run_bwd(d))


@pytest.mark.parametrize("g", ["one", "zero"])
def test_special_decays(g):
    d = inputs("bwd_bf16_b4_t4096", seed=4, B=1, T=260, H=2, g=g, S0="normal0.1", with_dO=True,
               with_dS_T=True)
    got = run_bwd(d)
    check(d, got)


@pytest.mark.parametrize("T,segments", [(1024, 4), (1100, 3)])
def test_segments(T, segments):
    d = inputs("bwd_bf16_b4_t4096", seed=6, B=1, T=T, H=2, S0="normal0.1", with_dO=True, with_dS_T=True)
    got = run_bwd(d, segments=segments)
    check(d, got)


def test_bf16_gradients():
    # gradients written in bf16: elementwise bound of the rounding on top of
    # the tolerance; dg stays fp32
    d = inputs("bwd_bf16_b4_t4096", seed=9, B=2, T=333, H=2, S0="normal0.1", with_dO=True, with_dS_T=True)
    got = run_bwd(d, out_dtype=torch.bfloat16)
    ref = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["dO"], d["S0"], d["dS_T"])
    for name, x, y in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        assert_close_bf16_out(x, y, TOL, name + "(bf16)")
    assert_close(got[3], ref[3], TOL, "dg")
    assert_close(got[4], ref[4], TOL, "dS0")


def test_backward_workload_sampled():
    # B=4, H=16, T=4096, S0 = 0, dS_T = 0; the oracle checks sampled (b, h).
    d = inputs("bwd_bf16_b4_t4096", seed=0, with_dO=True)
    got = run_bwd(d, S0=False, dS_T=False)
    bs, hs = [0, 3], [2, 13]
    sub = lambda x: x[np.ix_(bs, range(x.shape[1]), hs)]
    ref = oracle.backward(sub(d["q"]), sub(d["k"]), sub(d["v"]), sub(d["g"]), sub(d["dO"]))
    for name, x, y in zip(("dq", "dk", "dv", "dg"), got[:4], ref[:4]):
        assert_close(sub(x), y, TOL, name)
    for x in got[:4]:
        assert np.isfinite(x).all()


def test_longest_supported_sequence():
    """T = 131,072, the backward's limit of 1,024 chunks, on one head (the
    segment plan with every kernel at its largest chunk count)."""
    d = inputs("bwd_bf16_b4_t4096", seed=12, B=1, T=131_072, H=1, S0="normal0.1", with_dO=True,
               with_dS_T=True)
    print("case bwd T=131072", flush=True)
    got = run_bwd(d)
    ref = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["dO"], d["S0"], d["dS_T"], ckpt=1024)
    for name, x, y in zip(("dq", "dk", "dv", "dg", "dS0"), got, ref):
        assert_close(x, y, TOL, name)
