"""bench.py's algorithmic work counts reproduce the figures of the measurement spec for every
workload (FLOPs: only the needed triangles, KK^T and QK^T once per q/k head; bytes: inputs read
once, o in fp32 and the final state written once; decode: the state read and written once)."""
import bench


def test_prefill_counts():
    assert bench.prefill_flops(1, 4096, 16, 16, 128, 128, 64) == 9_207_873_536
    assert bench.prefill_bytes(1, 4096, 16, 16, 128, 128) == 85_196_800
    assert round(bench.prefill_flops(8, 8192, 16, 32, 128, 128, 64) / 1e9, 2) == 277.47
    assert bench.prefill_bytes(8, 8192, 16, 32, 128, 128, has_s0=True) == 2_189_426_688
    assert round(bench.prefill_flops(1, 262144, 16, 16, 128, 128, 64) / 1e9, 2) == 589.30
    assert bench.prefill_bytes(1, 262144, 16, 16, 128, 128) == 5_386_534_912


def test_prefill_flops_per_chunk_terms():
    # one full chunk of one head (C = 64, d = 128): 2 C^2 d for KK^T + QK^T, then the solve,
    # U and W, P Delta and the three state products
    C, d = 64, 128
    want = 2 * C * C * d + (C ** 3 - C) // 3 + C * (C - 1) * 2 * d + C * (C + 1) * d + 6 * C * d * d
    assert bench.prefill_flops(1, C, 1, 1, d, d, C) == want
    # a ragged last chunk is counted at its own length
    assert bench.prefill_flops(1, C + 1, 1, 1, d, d, C) == want + bench.prefill_flops(1, 1, 1, 1, d, d, C)


def test_decode_counts():
    state, total = bench.decode_bytes(256, 32, 32, 128, 128)
    assert state == 1_073_741_824
    assert total == 1_084_260_352
