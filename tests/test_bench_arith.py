"""The benchmark's algorithmic byte and flop counts (the numerators of its
roofline figures), checked against counts made from the tensor shapes."""
import numpy as np

import bench
import gen

H, DK, DV, CH = 16, 96, 192, 128


def test_prefill_bytes_from_shapes():
    B, T = 8, 2048
    q = k = B * T * H * DK * 2          # bf16 inputs
    v = B * T * H * DV * 2
    g = B * T * H * 4
    o = B * T * H * DV * 2              # bf16 output
    S_T = B * H * DK * DV * 4
    assert bench.fwd_bytes(B, T, 2, 2) == q + k + v + g + o + S_T == 312_475_648
    assert bench.fwd_bytes(1, 65536, 2, 2, s0=True) == 1 * 65536 * H * (2 * DK * 2 + DV * 2 + 4 + DV * 2) + 2 * H * DK * DV * 4


def test_flops_per_token_head():
    # dense 128-token chunk: Q K^T (C x dk), P V (C x dv), Q S (dk x dv), K^T V (dk x dv), 2 flops each
    assert bench.FWD_FLOP_PER_TH == 2 * CH * DK + 2 * CH * DV + 2 * DK * DV + 2 * DK * DV == 147_456
    # backward: scores and dO V^T (2 C dk + 2 C dv), dq, dk, dv intra (2 C dk + 2 C dk + 2 C dv), three
    # state products in the chunk gradients, the recomputed forward state and the reverse state gradient
    assert bench.BWD_FLOP_PER_TH == 2 * CH * (3 * DK + 2 * DV) + 10 * DK * DV == 356_352


def test_decode_bytes_from_shapes():
    n = 1280
    state = n * H * DK * DV * 4 * 2     # read and written in place
    io = n * H * (2 * DK * 2 + DV * 2 + 4 + DV * 4)    # bf16 q, k, v; fp32 g; fp32 o
    assert bench.decode_bytes(n) == state + io
    # 16-bit state: 96 x 192 int16 mantissas and 192 int32 exponents per
    # (sequence, head), read and written: 2 x 37,632 B
    assert bench.decode_bytes(n, q16=True) == n * H * (2 * 37_632) + io
    assert bench.decode_bytes(1, q16=True) // H == 76_804


def test_packed_bytes_match_the_workload():
    d = gen.make_packed_inputs("serve_prefill_16x2k8k", seed=0, with_pool=False)
    N, n_seq = int(d["cu_seqlens"][-1]), len(d["slot_idx"])
    assert N == int(np.sum(d["meta"]["lengths"])) and n_seq == 16
    per_token_head = 2 * DK * 2 + DV * 2 + 4 + DV * 2
    assert bench.packed_bytes(N, n_seq, 2, 2) == N * H * per_token_head + n_seq * H * DK * DV * 4


def test_mfma_ceilings():
    # bf16 prefill B=8 T=2048: 38.65 GFLOP take 15.46 us at 2.5 PFLOP/s, its
    # 312.5 MB take 39.06 us at 8 TB/s: the HBM roof allows 0.396 of the peak
    fwd = bench.mfma_ceiling(bench.FWD_FLOP_PER_TH * 8 * 2048 * H, bench.fwd_bytes(8, 2048, 2, 2), 2500.0)
    assert abs(fwd - (38_654_705_664 / 2.5e15) / (312_475_648 / 8e12)) < 1e-12
    assert 0.395 < fwd < 0.397
    # backward B=4 T=4096: 93.42 GFLOP (37.37 us) against 505.4 MB (63.18 us)
    bwd = bench.mfma_ceiling(bench.BWD_FLOP_PER_TH * 4 * 4096 * H, bench.bwd_bytes(4, 4096, 2, 2), 2500.0)
    assert 0.591 < bwd < 0.592
    # fp32 prefill B=1: 4.83 GFLOP at 157.3 TFLOP/s outlast its 76.8 MB: no cap
    f32 = bench.mfma_ceiling(bench.FWD_FLOP_PER_TH * 2048 * H, bench.fwd_bytes(1, 2048, 4, 4), 157.3)
    assert f32 == 1.0
    assert bench.mfma_ceiling(1.0, 0, 2500.0) == 1.0
