"""Seeded synthetic inputs for the Simple GLA mixer.

Shared by the tests, the smoke check and the benchmark, on both the oracle
side and the device side.  It holds none of the mixer's arithmetic: only the
input distributions and the host-side rounding of inputs to bfloat16.

Workloads (sizes from the pages: 16 heads, dk 96, dv 192 in "Diseño esencial
de Laplace 3B"; 16 chunks of 128 tokens in "Adaptaciones para AWS
Trainium2"; 1,280 concurrent decode sequences in "Resultados de
entrenamiento e inferencia").  The pages' training data (FineWeb-Edu) and
activations are not available; these Gaussian and log-sigmoid draws stand in
for them.

Every tensor comes from its own PCG64 stream seeded by
SeedSequence([workload id, tensor id, seed]).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "WORKLOADS", "TENSOR_IDS", "rng", "bf16_round", "bf16_bits",
    "logsigmoid", "make_g", "make_inputs", "make_decode_step",
    "make_decode_state", "make_packed_inputs",
]

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "g": 3, "S0": 4, "dO": 5, "u_head": 6,
              "dS_T": 7, "slot": 8, "len": 9, "gate": 10}

# name -> description.  "g" names the log-decay recipe (see make_g),
# "S0" the initial-state recipe ("zero" or "normal0.1": N(0, 0.1^2)).
WORKLOADS = {
    "fwd_f32_b1_t2048": dict(id=1, kind="fwd", B=1, T=2048, H=16, dk=96, dv=192,
                             dtype="f32", g="logsig_n4", S0="zero"),
    "fwd_bf16_b8_t2048": dict(id=2, kind="fwd", B=8, T=2048, H=16, dk=96, dv=192,
                              dtype="bf16", g="logsig_n4", S0="zero"),
    "fwd_bf16_b1_t65536": dict(id=3, kind="fwd", B=1, T=65536, H=16, dk=96, dv=192,
                               dtype="bf16", g="logsig_u28_head", S0="normal0.1"),
    "decode_1280x24x64": dict(id=4, kind="decode", B=1280, layers=24, steps=64, H=16,
                              dk=96, dv=192, dtype="bf16", g="logsig_n4",
                              S0="normal0.1"),
    "bwd_bf16_b4_t4096": dict(id=5, kind="bwd", B=4, T=4096, H=16, dk=96, dv=192,
                              dtype="bf16", g="logsig_n4", S0="zero"),
    # serving prefill: prompts of 2,048 to 8,192 tokens ("I risultati dichiarati
    # hanno limiti precisi") packed into one batch, states in a pool of 1,280
    # slots ("Resultados de entrenamiento e inferencia")
    "serve_prefill_16x2k8k": dict(id=6, kind="packed", n_seq=16, len_lo=2048,
                                  len_hi=8192, n_slots=1280, H=16, dk=96, dv=192,
                                  dtype="bf16", g="logsig_n4", S0="normal0.1"),
}


def rng(workload_id: int, tensor: str, seed: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([int(workload_id), TENSOR_IDS[tensor], int(seed)])
    return np.random.Generator(np.random.PCG64(ss))


def bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_round(x) -> np.ndarray:
    """Float32 array holding the bfloat16 (RNE) value of each element."""
    b = bf16_bits(x).astype(np.uint32) << 16
    return b.view(np.float32)


def logsigmoid(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return np.where(x >= 0, -np.log1p(np.exp(-np.abs(x))),
                    x - np.log1p(np.exp(-np.abs(x))))


def make_g(mode: str, shape, workload_id: int, seed: int = 0) -> np.ndarray:
    """Log-decay g (float32) of `shape` = (B, T, H) or (N, H).

    logsig_n4       : logsigmoid(z + 4), z ~ N(0, 1) per element (gamma ~ 0.98)
    logsig_u28_head : logsigmoid(u_h), u_h ~ U(2, 8), one draw per head, held
                      over every other index (slow and fast heads mixed)
    one             : g = 0       (gamma == 1, no decay)
    zero            : g = -inf    (gamma == 0, state forgets everything)
    """
    if mode == "logsig_n4":
        z = rng(workload_id, "g", seed).standard_normal(shape)
        return logsigmoid(z + 4.0).astype(np.float32)
    if mode == "logsig_u28_head":
        H = shape[-1]
        u = rng(workload_id, "u_head", seed).uniform(2.0, 8.0, size=H)
        return np.broadcast_to(logsigmoid(u).astype(np.float32), shape).copy()
    if mode == "one":
        return np.zeros(shape, np.float32)
    if mode == "zero":
        return np.full(shape, -np.inf, np.float32)
    raise ValueError(f"unknown log-decay recipe {mode!r}")


def _normal(workload_id, tensor, seed, shape, scale):
    x = rng(workload_id, tensor, seed).standard_normal(shape, dtype=np.float32)
    return x * np.float32(scale)


def make_inputs(workload: str, seed: int = 0, B=None, T=None, H=None, dk=None,
                dv=None, g=None, S0=None, dtype=None, with_dO=False,
                with_dS_T=False, with_gate=False) -> dict:
    """Inputs of a prefill/backward workload as float32 numpy arrays.

    Keyword arguments override the workload's sizes or recipes (reduced
    shapes for parity tests).  For bf16 workloads q, k, v, dO and the gate
    hold bf16-representable values (S0 and dS_T stay float32).
    """
    w = dict(WORKLOADS[workload])
    for key, val in (("B", B), ("T", T), ("H", H), ("dk", dk), ("dv", dv),
                     ("g", g), ("S0", S0), ("dtype", dtype)):
        if val is not None:
            w[key] = val
    wid, Bn, Tn, Hn, K, V = w["id"], w["B"], w["T"], w["H"], w["dk"], w["dv"]
    sc = 1.0 / math.sqrt(K)
    out = {
        "q": _normal(wid, "q", seed, (Bn, Tn, Hn, K), sc),
        "k": _normal(wid, "k", seed, (Bn, Tn, Hn, K), sc),
        "v": _normal(wid, "v", seed, (Bn, Tn, Hn, V), sc),
        "g": make_g(w["g"], (Bn, Tn, Hn), wid, seed),
    }
    if w["S0"] == "zero":
        out["S0"] = None
    elif w["S0"] == "normal0.1":
        out["S0"] = _normal(wid, "S0", seed, (Bn, Hn, K, V), 0.1)
    else:
        raise ValueError(f"unknown initial-state recipe {w['S0']!r}")
    if with_dO:
        out["dO"] = _normal(wid, "dO", seed, (Bn, Tn, Hn, V), 1.0)
    if with_dS_T:
        out["dS_T"] = _normal(wid, "dS_T", seed, (Bn, Hn, K, V), 0.1)
    if with_gate:
        # the output gate of the fused projection, [B, T, H, dv]: N(0, 1)
        out["gate"] = _normal(wid, "gate", seed, (Bn, Tn, Hn, V), 1.0)
    if w["dtype"] == "bf16":
        for key in ("q", "k", "v", "dO", "gate"):
            if key in out:
                out[key] = bf16_round(out[key])
    out["meta"] = w
    return out


def make_decode_state(n_seq: int, H=16, dk=96, dv=192, seed=0, workload_id=4):
    """Initial decode state, N(0, 0.1^2) per element, float32 [n_seq, H, dk, dv]."""
    return _normal(workload_id, "S0", seed, (n_seq, H, dk, dv), 0.1)


def make_decode_step(n_seq: int, step: int, H=16, dk=96, dv=192, seed=0,
                     dtype="bf16", g="logsig_n4", workload_id=4) -> dict:
    """One decode token per sequence for step `step`: q, k [N,H,dk], v [N,H,dv], g [N,H]."""
    s = seed * 100003 + step
    sc = 1.0 / math.sqrt(dk)
    out = {
        "q": _normal(workload_id, "q", s, (n_seq, H, dk), sc),
        "k": _normal(workload_id, "k", s, (n_seq, H, dk), sc),
        "v": _normal(workload_id, "v", s, (n_seq, H, dv), sc),
        "g": make_g(g, (n_seq, H), workload_id, s),
    }
    if dtype == "bf16":
        for key in ("q", "k", "v"):
            out[key] = bf16_round(out[key])
    return out


def make_packed_inputs(workload: str = "serve_prefill_16x2k8k", seed: int = 0, lengths=None,
                       n_slots=None, H=None, dtype=None, g=None, with_pool=True) -> dict:
    """Sequences of different lengths packed along one token axis.

    lengths    : per-sequence token counts (default: n_seq draws, uniform
                 integers in [len_lo, len_hi])
    returns q, k [N, H, dk], v [N, H, dv], g [N, H] (float32 arrays, bf16
    values for bf16 workloads), cu_seqlens int32 [n_seq + 1], slot_idx int32
    [n_seq] (distinct slots of an n_slots pool, in random order) and, with
    with_pool, the pool's initial states float32 [n_slots, H, dk, dv] drawn
    N(0, 0.1^2).
    """
    w = dict(WORKLOADS[workload])
    for key, val in (("n_slots", n_slots), ("H", H), ("dtype", dtype), ("g", g)):
        if val is not None:
            w[key] = val
    wid, Hn, K, V = w["id"], w["H"], w["dk"], w["dv"]
    if lengths is None:
        lengths = rng(wid, "len", seed).integers(w["len_lo"], w["len_hi"] + 1, size=w["n_seq"])
    lengths = np.asarray(lengths, dtype=np.int64)
    n_seq = len(lengths)
    if n_seq > w["n_slots"]:
        raise ValueError(f"{n_seq} sequences do not fit {w['n_slots']} slots")
    cu = np.zeros(n_seq + 1, np.int64)
    cu[1:] = np.cumsum(lengths)
    N = int(cu[-1])
    sc = 1.0 / math.sqrt(K)
    out = {
        "q": _normal(wid, "q", seed, (N, Hn, K), sc),
        "k": _normal(wid, "k", seed, (N, Hn, K), sc),
        "v": _normal(wid, "v", seed, (N, Hn, V), sc),
        "g": make_g(w["g"], (N, Hn), wid, seed),
        "cu_seqlens": cu.astype(np.int32),
        "slot_idx": rng(wid, "slot", seed).permutation(w["n_slots"])[:n_seq].astype(np.int32),
    }
    if with_pool:
        out["pool"] = _normal(wid, "S0", seed, (w["n_slots"], Hn, K, V), 0.1)
    if w["dtype"] == "bf16":
        for key in ("q", "k", "v"):
            out[key] = bf16_round(out[key])
    w["lengths"] = lengths
    out["meta"] = w
    return out
