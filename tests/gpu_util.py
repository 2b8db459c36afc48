"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import numpy as np
import torch

import gen
import oracle


def dev():
    return torch.device("cuda", 0)


def to_dev(x, dtype):
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev()).to(dtype)


def to_np(t):
    return None if t is None else t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    """max |got - ref| / rms(ref), in float64."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(got - ref)) / rms) if rms > 0 else float(np.max(np.abs(got - ref)))


def assert_close(got, ref, tol, name):
    e = rel_err(got, ref)
    print(f"  {name}: max|err|/rms = {e:.3e} (tol {tol:.0e})", flush=True)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert e <= tol, f"{name}: max|err|/rms(ref) = {e:.3e} > {tol:.1e}"
    return e


def assert_close_bf16_out(got, ref, tol, name):
    """bf16 outputs: |got - ref| <= tol*rms(ref) + 2^-8 |ref| elementwise."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    bound = tol * rms + 2.0 ** -8 * np.abs(ref)
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{name}: {bad.sum()} elements outside the bf16-output bound"


def inputs(workload, seed=0, **kw):
    return gen.make_inputs(workload, seed=seed, **kw)


def check_q16_state(m, e, m_ref, e_ref, S_ref, name):
    """Stored state against the oracle's: equal exponents except at a
    threshold, every value within one quantum of the coarser exponent."""
    M = np.abs(S_ref).max(axis=-2)
    diff = e != e_ref
    if diff.any():
        r = M[diff] * np.exp2(-e_ref[diff].astype(np.float64))
        dist = np.minimum.reduce([np.abs(r / t - 1) for t in (16383.75, 16384.0, 32767.5)])
        assert np.all(dist < 1e-6), f"{name}: exponents differ away from a threshold"
        assert np.all(np.abs(e[diff].astype(np.int64) - e_ref[diff]) == 1)
    quantum = np.exp2(np.maximum(e, e_ref).astype(np.float64))[..., None, :]
    gap = np.abs(oracle.q16_decode(m, e) - oracle.q16_decode(m_ref, e_ref))
    assert np.all(gap <= quantum), f"{name}: {np.sum(gap > quantum)} values more than a quantum apart"
    same_e = np.broadcast_to(~diff[..., None, :], m.shape)
    moved = np.mean(m[same_e] != m_ref[same_e])
    print(f"  {name}: {diff.sum()} exponents differ, {moved:.2e} of mantissas differ by 1", flush=True)
