"""The seeded workloads and their accounting: the bytes, update and flop
counts that bench.py divides by, checked against the per-config figures
derived from the method (state read and written once per live (sequence,
v-head), every token's activations once), and the input recipe (shapes,
padding, slot sets, value distributions)."""
import numpy as np
import pytest

from linear_attention_recurrent_gating_amd import workloads as W

KIB64 = 128 * 128 * 4   # one fp32 K x V tile at K = V = 128


@pytest.mark.parametrize("wl,expect_bytes,expect_updates", [
    (W.TINY_F32, 68_712, 8),
    (W.QWEN3NEXT_B64, 270_017_024, 2_048),
    (W.DECODE_B512, 2_160_134_400, 16_384),
    (W.DECODE_B512_SHARD, 540_035_136, 4_096),
    (W.SPEC_VERIFY, 1_458_400_004, 14_720),
], ids=lambda x: x.name if isinstance(x, W.Workload) else None)
def test_algorithmic_bytes_and_updates(wl, expect_bytes, expect_updates):
    inp = W.make_host_inputs(wl)
    assert W.algorithmic_bytes(inp) == expect_bytes
    assert W.active_updates(inp) == expect_updates


def test_decode_bytes_per_update_is_mostly_state():
    inp = W.make_host_inputs(W.DECODE_B512)
    params = 32 * 4 * 2 + 512 * 4          # A_log, dt_bias, slot indices
    per_update = (W.algorithmic_bytes(inp) - params) / W.active_updates(inp)
    assert per_update == 131_844
    assert 2 * KIB64 / per_update > 0.994


def test_spec_verify_bytes_by_parts():
    """115 live sequences x 32 heads: one read, four intermediates and one
    final write per tile; 460 tokens of bf16 q, k (16 heads), v, out (32
    heads) and a, b; A_log, dt_bias, slot indices and cu_seqlens."""
    inp = W.make_host_inputs(W.SPEC_VERIFY)
    live = int((inp.state_idx >= 0).sum())
    assert live == 115
    tokens = 4 * live
    act = tokens * (2 * 16 * 128 * 2 + 2 * 32 * 128 * 2 + 2 * 32 * 2)
    params = 32 * 4 * 2 + 128 * 4 + 129 * 4
    assert W.algorithmic_bytes(inp) == live * 32 * KIB64 * 6 + act + params
    assert W.algorithmic_bytes(inp, final_writeback=False) == live * 32 * KIB64 * 5 + act + params
    # bf16 state storage halves every state byte and nothing else
    assert W.algorithmic_bytes(inp, state_bytes=2) == live * 32 * KIB64 * 3 + act + params


def test_varlen_long_lengths_and_bytes():
    inp = W.make_host_inputs(W.VARLEN_LONG)
    assert inp.lengths.min() >= 64 and inp.lengths.max() <= 2048
    assert np.array_equal(inp.cu_seqlens[1:], np.cumsum(inp.lengths))
    total = int(inp.lengths.sum())
    assert W.active_updates(inp) == total * 32
    params = 32 * 8 + 8 * 4 + 9 * 4
    assert W.algorithmic_bytes(inp) == 8 * 32 * KIB64 * 2 + total * 24_704 + params


def test_recurrent_flops():
    """Seven flops per state element and token: one decay multiply, two
    multiply-adds of S^T k, two of the rank-1 update, two of S^T q."""
    for wl in (W.DECODE_B512, W.SPEC_VERIFY, W.VARLEN_LONG):
        inp = W.make_host_inputs(wl)
        assert W.recurrent_flops(inp) == W.active_updates(inp) * 128 * 128 * 7


def _chunk_products(c, K, V):
    """(m, n, depth) of each dense product of one chunk of c tokens."""
    return [(c, c, K),    # key-key Gram matrix
            (c, c, K),    # query-key products
            (c, V, K),    # keys times the chunk-start state
            (c, V, K),    # queries times the chunk-start state
            (c, V, c),    # triangular factor times the right-hand side
            (c, V, c),    # masked query-key matrix times U
            (K, V, c)]    # state update: keys^T times U


def test_chunked_flops_counts_every_product():
    wl = W.Workload("one_chunk", 9, 1, 64, 1, 1, 128, 128, W.ACT_BF16, 1, 0.05)
    inp = W.make_host_inputs(wl)
    dense = sum(2 * m * n * d for m, n, d in _chunk_products(64, 128, 128))
    inverse = (2 * 64 ** 3) // 3          # c^3 / 3 multiply-adds of a triangular inverse
    assert W.chunked_flops(inp) == dense + inverse
    # a ragged tail chunk is counted at its own length
    wl2 = wl.with_(name="chunk_and_tail", tokens_per_seq=64 + 10)
    inp2 = W.make_host_inputs(wl2)
    tail = sum(2 * m * n * d for m, n, d in _chunk_products(10, 128, 128)) + (2 * 10 ** 3) // 3
    assert W.chunked_flops(inp2) == dense + inverse + tail
    # padded sequences do no work
    wl3 = wl.with_(name="padded", num_seqs=2, num_slots=2, num_padded=1)
    assert W.chunked_flops(W.make_host_inputs(wl3)) == dense + inverse


def test_input_recipe():
    inp = W.make_host_inputs(W.DECODE_B512)
    # q, k, v, a, b ~ N(0, 1), rounded to bf16
    for name in ("q", "k", "v", "a", "b"):
        x = getattr(inp, name)
        tol = 5.0 / np.sqrt(x.size)           # five standard errors
        assert abs(float(x.mean())) < tol and abs(float(x.std()) - 1.0) < tol, name
        assert np.array_equal(W.round_to_bf16(x)[1], x), f"{name} is not bf16-exact"
    # dt_bias ~ N(0, 0.5), A_log = log U[1, 16] per v-head
    assert inp.dt_bias.shape == (32,) and np.all(np.abs(inp.dt_bias) < 3.0)
    assert np.all(inp.A_log >= 0.0) and np.all(inp.A_log <= np.log(16.0) + 1e-6)
    # distinct slots drawn from the whole pool
    assert len(set(inp.state_idx.tolist())) == 512 and inp.state_idx.max() < 4096
    # the tiny case uses the fixed slots [2, 0]
    assert W.make_host_inputs(W.TINY_F32).state_idx.tolist() == [2, 0]
    # spec verify: 13 padded sequences, the rest distinct
    sv = W.make_host_inputs(W.SPEC_VERIFY)
    assert int((sv.state_idx == -1).sum()) == 13
    live = sv.state_idx[sv.state_idx >= 0]
    assert len(set(live.tolist())) == live.size
    # weak decay: A_log = log U[1e-3, 1e-2]
    weak = W.make_host_inputs(W.SPEC_VERIFY.with_(decay="weak"))
    assert np.all(np.exp(weak.A_log) >= 1e-3) and np.all(np.exp(weak.A_log) <= 1e-2)


def test_inputs_are_reproducible():
    a, b = W.make_host_inputs(W.SPEC_VERIFY), W.make_host_inputs(W.SPEC_VERIFY)
    for name in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "state_idx", "cu_seqlens"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    p0, p1 = W.make_pool_host(W.TINY_F32), W.make_pool_host(W.TINY_F32)
    assert np.array_equal(p0, p1) and abs(float(p0.std()) - 0.1) < 0.02


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it says so and exits 2
    before touching a device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_kernel_names_are_kernel_symbols():
    """The kernel named in the bench line (and used to find its profiles) is
    a kernel defined in the HIP sources, for every family and token mode."""
    import glob
    import os
    import re
    import sys
    from types import SimpleNamespace
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    src = "".join(open(p).read() for p in
                  glob.glob(os.path.join(root, "linear_attention_recurrent_gating_amd", "csrc", "*.hip")))
    for family in (1, 2, 3, 4):
        for multi in (0, 1):
            name = bench.kernel_name(SimpleNamespace(kernel_family=family, multi_token=multi))
            assert re.search(r"__global__[^;{]*\b" + name + r"\s*\(", src), name
