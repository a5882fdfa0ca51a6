"""HIP path against the CPU oracle, element by element, on seeded inputs.

Small cases run the oracle on everything and span several wavefront tiles,
GQA groups, K != V, chunk boundaries of the token loop and ragged tails.  The
five named workloads run at their full sizes in the launch configuration the
benchmark times; where the oracle would be slow it checks a sample of
sequences one by one, and properties (untouched slots, padded rows) are
checked over everything."""
import numpy as np
import pytest

from gpu_helpers import (TOL_STATE_GUARD, announce, check_vs_oracle, live_rows, oracle_on_seqs,
                         rel_err, run_gpu, to_layout, to_np, tol_for)
from linear_attention_recurrent_gating_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


def full_check(wl, dev, block_v=0, waves=0, check_inter=True, family=0, block_k=0, layout="KV"):
    """Whole-batch parity: out, final states, intermediates, untouched rows."""
    import torch
    announce(f"{wl.name} B={wl.num_seqs} H={wl.num_k_heads}/{wl.num_v_heads} K={wl.head_k_dim} "
             f"V={wl.head_v_dim} act={wl.act} layout={layout} family={family} bv={block_v} "
             f"bk={block_k} waves={waves}")
    inp = W.make_host_inputs(wl)
    pool_np = to_layout(W.make_pool_host(wl), layout)
    pool = torch.from_numpy(pool_np).to(dev)
    out, inter = run_gpu(inp, pool, dev, block_v=block_v, waves_per_group=waves,
                         kernel_family=family, block_k=block_k, layout=layout)
    seqs = np.arange(wl.num_seqs)
    ref_pool_rows = pool_np[np.maximum(inp.state_idx, 0)]
    o_ref, s_ref, i_ref, rows = oracle_on_seqs(inp, ref_pool_rows, seqs,
                                               intermediates=wl.intermediates, layout=layout)
    tol = tol_for(wl)
    live, dead = live_rows(inp)
    out_np = to_np(out)
    e_out = rel_err(out_np[live], o_ref[live])
    assert e_out <= tol, f"out error {e_out:.3e} > {tol}"
    assert np.all(np.isnan(out_np[dead])), "padded sequences wrote outputs"
    pool_after = pool.cpu().numpy()
    lv = inp.state_idx >= 0
    e_state = rel_err(pool_after[inp.state_idx[lv]], s_ref[lv])
    assert e_state <= min(tol, TOL_STATE_GUARD), f"state error {e_state:.3e}"
    untouched = np.setdiff1d(np.arange(wl.num_slots), inp.state_idx[lv])
    assert np.array_equal(pool_after[untouched], pool_np[untouched]), "untouched slots changed"
    if wl.intermediates and check_inter:
        inter_np = inter.cpu().numpy()
        e_inter = rel_err(inter_np[live], i_ref[live])
        assert e_inter <= min(tol, TOL_STATE_GUARD), f"intermediate error {e_inter:.3e}"
        assert np.all(np.isnan(inter_np[dead])), "padded sequences wrote intermediates"
        # the last token's intermediate is the final state, bitwise
        ends = np.cumsum(inp.lengths) - 1
        for i in np.nonzero(lv & (inp.lengths > 0))[0]:
            assert np.array_equal(inter_np[ends[i]], pool_after[inp.state_idx[i]])
    return e_out, e_state


SMALL = [
    W.Workload("k32v32_g2_f32_b5", 21, 5, 1, 2, 4, 32, 32, W.ACT_F32, 9, 0.1),
    W.Workload("k64v64_g2_bf16_b7", 22, 7, 1, 2, 4, 64, 64, W.ACT_BF16, 12, 0.1),
    W.Workload("k128v128_g2_bf16_b9", 23, 9, 1, 4, 8, 128, 128, W.ACT_BF16, 16, 0.05),
    W.Workload("k128v128_g2_f32_b9", 24, 9, 1, 4, 8, 128, 128, W.ACT_F32, 16, 0.05),
    W.Workload("k32v64_g1_f32_t3", 25, 4, 3, 3, 3, 32, 64, W.ACT_F32, 6, 0.1),
    W.Workload("k64v128_g4_bf16_t2", 26, 3, 2, 1, 4, 64, 128, W.ACT_BF16, 5, 0.1),
    W.Workload("k256v128_g2_bf16_b3", 27, 3, 1, 2, 4, 256, 128, W.ACT_BF16, 4, 0.05),
    W.Workload("k128v256_g2_f32_b3", 28, 3, 1, 1, 2, 128, 256, W.ACT_F32, 4, 0.05),
    W.Workload("k128v128_g3_bf16_b4", 29, 4, 1, 2, 6, 128, 128, W.ACT_BF16, 6, 0.05),
    W.Workload("k128v128_f32_t17_inter", 30, 3, 17, 2, 4, 128, 128, W.ACT_F32, 5, 0.05,
               intermediates=True),
    W.Workload("varlen_0_40_bf16", 31, 6, 1, 2, 4, 128, 128, W.ACT_BF16, 8, 0.05, varlen=True,
               len_range=(0, 40)),
    W.Workload("varlen_pad_inter_f32", 32, 9, 1, 2, 4, 64, 64, W.ACT_F32, 12, 0.1, varlen=True,
               len_range=(1, 20), num_padded=3, intermediates=True),
    W.Workload("k128v128_weak_decay_t9", 33, 4, 9, 2, 4, 128, 128, W.ACT_F32, 5, 0.05,
               decay="weak"),
    W.Workload("tiny_fp32_weak_decay", 0, 2, 1, 2, 4, 32, 32, W.ACT_F32, 4, 0.1,
               fixed_slots=(2, 0), decay="weak"),
]


def test_tiny_fp32(dev):
    full_check(W.TINY_F32, dev)


ROW_SPLIT_PAIRS = [(K, V) for K in (32, 64, 128, 256) for V in (32, 64, 128, 256)]


@pytest.mark.parametrize("K,V", ROW_SPLIT_PAIRS, ids=lambda x: str(x))
def test_single_token_all_head_dims(dev, K, V):
    """Single-token decode over every supported (K, V): AUTO's row-split
    tile for each (32 rows per lane with fp32 state, 8 wavefronts per head
    at K = V = 256), bf16 and fp32 activations."""
    for act, seed in ((W.ACT_BF16, 60), (W.ACT_F32, 61)):
        wl = W.Workload(f"decode_k{K}_v{V}_{act}", seed + K + V, 5, 1, 2, 4, K, V, act, 8, 0.05,
                        num_padded=1)
        full_check(wl, dev)


@pytest.mark.parametrize("K,V", [(32, 32), (64, 128), (128, 32), (128, 64), (128, 128),
                                 (256, 32), (256, 64)], ids=lambda x: str(x))
def test_row_split_eight_rows_per_lane(dev, K, V):
    """Row split with 8 state rows per lane (block_k = 8 * rows per
    instruction) and with one head per workgroup."""
    import linear_attention_recurrent_gating_amd as gdn
    rg = 64 // (V // 4)
    for act, seed in ((W.ACT_BF16, 63), (W.ACT_F32, 64)):
        wl = W.Workload(f"rows8_k{K}_v{V}_{act}", seed + K + V, 5, 1, 2, 4, K, V, act, 8, 0.05,
                        num_padded=1)
        if K >= 8 * rg and K // (8 * rg) <= 8:
            full_check(wl, dev, family=gdn.GDN_KERNEL_ROW_SPLIT, block_k=8 * rg)
        kw = max(1, K // (16 * rg))
        full_check(wl, dev, family=gdn.GDN_KERNEL_ROW_SPLIT, waves=kw)


@pytest.mark.parametrize("K,V", [(64, 64), (64, 128), (128, 64), (128, 128), (128, 256),
                                 (256, 128)], ids=lambda x: str(x))
def test_row_split_sixteen_rows_per_lane(dev, K, V):
    """Row split with 16 state rows per lane (block_k = 16 * rows per
    instruction): the single-token instance for bf16 state at large grids
    outside K = V = 128, and for fp32 intermediates at K or V = 64."""
    import linear_attention_recurrent_gating_amd as gdn
    rg = 64 // (V // 4)
    bk = 16 * rg
    for act, seed in ((W.ACT_BF16, 67), (W.ACT_F32, 68)):
        wl = W.Workload(f"rows16_k{K}_v{V}_{act}", seed + K + V, 5, 1, 2, 4, K, V, act, 8, 0.05,
                        num_padded=1)
        full_check(wl, dev, family=gdn.GDN_KERNEL_ROW_SPLIT, block_k=bk)


# Every (K, V) with such an instance: block_k = 32 * 64 / (V / 4) must not
# exceed K (which rules out (32, 32), (64, 64) and (128, 32)).
@pytest.mark.parametrize("K,V", [(128, 64), (128, 128), (256, 64), (256, 128)],
                         ids=lambda x: str(x))
def test_row_split_thirty_two_rows_per_lane(dev, K, V):
    """Row split with 32 state rows per lane (block_k = 32 * rows per
    instruction): the instance chosen for large fp32 grids at K = V = 128."""
    import linear_attention_recurrent_gating_amd as gdn
    rg = 64 // (V // 4)
    bk = 32 * rg
    assert bk <= K and K // bk <= 8
    for act, seed in ((W.ACT_BF16, 65), (W.ACT_F32, 66)):
        wl = W.Workload(f"rows32_k{K}_v{V}_{act}", seed + K + V, 5, 1, 2, 4, K, V, act, 8, 0.05,
                        num_padded=1)
        full_check(wl, dev, family=gdn.GDN_KERNEL_ROW_SPLIT, block_k=bk)


@pytest.mark.parametrize("K,V", ROW_SPLIT_PAIRS, ids=lambda x: str(x))
def test_token_loop_all_head_dims(dev, K, V):
    """Several tokens per sequence over every (K, V), with intermediates:
    AUTO's kernel (the row split's token loop, or column tiles at
    K = V = 256) and the column tiles, across the 16-token staging chunk."""
    for act, seed, T in ((W.ACT_BF16, 80, 3), (W.ACT_F32, 81, 18)):
        wl = W.Workload(f"tokens_k{K}_v{V}_{act}_t{T}", seed + K + V, 3, T, 2, 4, K, V, act, 6, 0.05,
                        num_padded=1, intermediates=True)
        full_check(wl, dev)
        full_check(wl, dev, family=1)


ROWS_TOKEN_CASES = [
    W.Workload("rows_t5_f32", 70, 3, 5, 2, 4, 128, 128, W.ACT_F32, 5, 0.05, intermediates=True),
    W.Workload("rows_t20_bf16", 71, 3, 20, 2, 4, 128, 128, W.ACT_BF16, 5, 0.05,
               intermediates=True, num_padded=1),
    W.Workload("rows_varlen", 72, 7, 1, 2, 4, 128, 128, W.ACT_BF16, 9, 0.05, varlen=True,
               len_range=(0, 40), num_padded=2, intermediates=True),
    W.Workload("rows_k64_v128_g3", 73, 3, 7, 2, 6, 64, 128, W.ACT_F32, 4, 0.05,
               intermediates=True),
    W.Workload("rows_k256_v64", 74, 2, 17, 1, 2, 256, 64, W.ACT_BF16, 3, 0.05),
    W.Workload("rows_k32_v32_t33", 75, 4, 33, 2, 2, 32, 32, W.ACT_F32, 5, 0.05,
               intermediates=True),
    W.Workload("rows_k128_v256", 76, 2, 3, 1, 2, 128, 256, W.ACT_F32, 3, 0.05,
               intermediates=True),
]


@pytest.mark.parametrize("wl", ROWS_TOKEN_CASES, ids=lambda w: w.name)
def test_row_split_token_loop(dev, wl):
    """The row-split kernel over several tokens per sequence (fixed T and
    cu_seqlens with empty and padded sequences, chunk boundaries at 16)."""
    import linear_attention_recurrent_gating_amd as gdn
    full_check(wl, dev, family=gdn.GDN_KERNEL_ROW_SPLIT)


@pytest.mark.parametrize("rpl", [8, 16, 32])
def test_row_split_token_loop_rows_per_lane(dev, rpl):
    """Every rows-per-lane instance of the token loop (block_k = rpl * 2 at
    V = 128), with intermediates."""
    import linear_attention_recurrent_gating_amd as gdn
    wl = W.Workload(f"rows_tokens_rpl{rpl}", 77 + rpl, 3, 6, 2, 4, 128, 128, W.ACT_BF16, 5, 0.05,
                    intermediates=True, num_padded=1)
    full_check(wl, dev, family=gdn.GDN_KERNEL_ROW_SPLIT, block_k=2 * rpl)


def test_row_split_chain_bitwise(dev):
    """A T-token row-split call equals T chained single-token row-split
    (decode) calls bit for bit: the token loop repeats the single-token
    kernel's arithmetic in the same order."""
    import torch
    import linear_attention_recurrent_gating_amd as gdn
    announce("row-split chain bitwise")
    wl = W.Workload("rows_chain", 78, 3, 6, 2, 4, 128, 128, W.ACT_BF16, 5, 0.05, intermediates=True)
    inp = W.make_host_inputs(wl)
    pool_np = W.make_pool_host(wl)
    fam = gdn.GDN_KERNEL_ROW_SPLIT
    pool_multi = torch.from_numpy(pool_np).to(dev)
    out_multi, inter = run_gpu(inp, pool_multi, dev, kernel_family=fam, block_k=32)
    pool_chain = torch.from_numpy(pool_np).to(dev)
    T = wl.tokens_per_seq
    for t in range(T):
        rows = np.arange(wl.num_seqs) * T + t
        step = W.HostInputs(wl.with_(tokens_per_seq=1, intermediates=False), inp.q[rows],
                            inp.k[rows], inp.v[rows], inp.a[rows], inp.b[rows], inp.A_log,
                            inp.dt_bias, inp.state_idx, None, np.ones(wl.num_seqs, np.int64),
                            {n: x[rows] for n, x in inp.bits.items()})
        out_t, _ = run_gpu(step, pool_chain, dev, kernel_family=fam, block_k=32)
        assert torch.equal(out_t, out_multi[torch.from_numpy(rows).to(dev)]), f"out differs at t={t}"
        for i in range(wl.num_seqs):
            assert torch.equal(pool_chain[int(inp.state_idx[i])], inter[int(rows[i])]), \
                f"state differs at t={t}, seq {i}"
    assert torch.equal(pool_chain, pool_multi)


def test_decode_kernel_families_agree(dev):
    """The row-split and column-tile single-token kernels differ only in the
    order of their fp32 reductions."""
    import torch
    announce("decode kernel families")
    wl = W.Workload("families", 62, 16, 1, 4, 8, 128, 128, W.ACT_F32, 20, 0.05)
    inp = W.make_host_inputs(wl)
    pool_np = W.make_pool_host(wl)
    p_rows = torch.from_numpy(pool_np).to(dev)
    p_cols = torch.from_numpy(pool_np).to(dev)
    o_rows, _ = run_gpu(inp, p_rows, dev)
    o_cols, _ = run_gpu(inp, p_cols, dev, block_v=32)
    assert rel_err(to_np(o_rows), to_np(o_cols)) <= 1e-5
    assert rel_err(p_rows.cpu().numpy(), p_cols.cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_small(dev, wl):
    full_check(wl, dev)


@pytest.mark.parametrize("t", [1, 5, 20])
def test_tile_overrides(dev, t):
    """Every tile width and workgroup size of the table on one shape."""
    for bv in (8, 16, 32, 64):
        for waves in (1, 2, 4, 8):
            units = 2 * (128 // bv)
            if units % waves:
                continue
            wl = W.Workload(f"override_t{t}", 40 + t, 3, t, 2, 4, 128, 128, W.ACT_F32, 5, 0.05,
                            intermediates=(t == 5))
            full_check(wl, dev, block_v=bv, waves=waves)


def test_qwen3next_b64(dev):
    full_check(W.QWEN3NEXT_B64, dev)


@pytest.mark.parametrize("family", [0, 1], ids=["auto_row_split", "column_tiles"])
def test_spec_verify_b128_t4(dev, family):
    full_check(W.SPEC_VERIFY, dev, family=family)


def test_spec_verify_weak_decay(dev):
    full_check(W.SPEC_VERIFY.with_(name="spec_verify_weak", decay="weak", seed=44), dev)


@pytest.mark.parametrize("family", [0, 1, 2], ids=["auto_chunked", "column_tiles", "row_split"])
def test_varlen_long(dev, family):
    """The long-varlen workload: AUTO takes the chunked kernel there (no
    intermediate states, long sequences); the per-token kernels (column
    tiles, and the row split's token loop over 2048-token sequences) are
    checked on it too."""
    full_check(W.VARLEN_LONG, dev, family=family)


@pytest.mark.parametrize("family", [0, 1, 2], ids=["auto_chunked", "column_tiles", "row_split"])
def test_varlen_long_weak_decay(dev, family):
    full_check(W.VARLEN_LONG.with_(name="varlen_long_weak", decay="weak", seed=45), dev,
               family=family)


def check_full_size_decode(wl, dev, layout):
    """Full-size decode in the benchmark's launch configuration, against the
    oracle on every sequence: all B x H_v (sequence, v-head) units, every
    output row and every element of every used state tile.  Untouched slots
    are checked bitwise over the whole pool."""
    import torch
    announce(f"{wl.name} full size, layout {layout}, all {wl.num_seqs} sequences")
    inp = W.make_host_inputs(wl)
    pool = W.make_pool_torch(wl, dev)
    if layout == "VK":
        pool = pool.transpose(-1, -2).contiguous()
    pool0 = pool.clone()
    slots = torch.from_numpy(inp.state_idx).long().to(dev)
    rows0 = pool0[slots].cpu().numpy()
    out, _ = run_gpu(inp, pool, dev, layout=layout)
    seqs = np.arange(wl.num_seqs)
    o_ref, s_ref, _, rows = oracle_on_seqs(inp, rows0, seqs, layout=layout)
    assert np.array_equal(rows, np.arange(inp.num_tokens))
    e_out = rel_err(to_np(out), o_ref)
    assert e_out <= tol_for(wl), f"out error {e_out:.3e}"
    e_state = rel_err(pool[slots].cpu().numpy(), s_ref)
    assert e_state <= TOL_STATE_GUARD, f"state error {e_state:.3e}"
    changed = (pool != pool0).flatten(1).any(dim=1).cpu().numpy()
    assert set(np.nonzero(changed)[0]) <= set(inp.state_idx.tolist()), "untouched slot changed"
    assert not torch.isnan(out).any(), "an output row was not written"
    print(f"{wl.name} {layout}: out {e_out:.2e} state {e_state:.2e} over {wl.num_seqs} sequences")


@pytest.mark.parametrize("wl", [W.DECODE_B512, W.DECODE_B512_SHARD], ids=lambda w: w.name)
def test_decode_b512_full_size(dev, wl):
    check_full_size_decode(wl, dev, "KV")


def test_chain_equals_multi_token_bitwise(dev):
    """A T-token call equals T chained one-token calls bit for bit (same fp32
    state both ways), and each chained state equals the intermediate.  The
    one-token calls pass cu_seqlens, so both sides run the token-loop kernel
    (test_row_split_chain_bitwise chains through the single-token kernel)."""
    import torch
    announce("chain bitwise")
    wl = W.Workload("chain", 50, 3, 6, 2, 4, 128, 128, W.ACT_BF16, 5, 0.05, intermediates=True)
    inp = W.make_host_inputs(wl)
    pool_np = W.make_pool_host(wl)
    pool_multi = torch.from_numpy(pool_np).to(dev)
    out_multi, inter = run_gpu(inp, pool_multi, dev)
    pool_chain = torch.from_numpy(pool_np).to(dev)
    T = wl.tokens_per_seq
    for t in range(T):
        rows = np.arange(wl.num_seqs) * T + t
        step = W.HostInputs(wl.with_(tokens_per_seq=1, intermediates=False, varlen=True),
                            inp.q[rows], inp.k[rows], inp.v[rows], inp.a[rows], inp.b[rows],
                            inp.A_log, inp.dt_bias, inp.state_idx,
                            np.arange(wl.num_seqs + 1, dtype=np.int32),
                            np.ones(wl.num_seqs, np.int64),
                            {n: x[rows] for n, x in inp.bits.items()})
        out_t, _ = run_gpu(step, pool_chain, dev)
        assert torch.equal(out_t, out_multi[torch.from_numpy(rows).to(dev)]), f"out differs at t={t}"
        for i in range(wl.num_seqs):
            assert torch.equal(pool_chain[int(inp.state_idx[i])], inter[int(rows[i])]), \
                f"state differs at t={t}, seq {i}"
    assert torch.equal(pool_chain, pool_multi)


def test_chain_through_decode_kernel(dev):
    """T chained single-token decode calls (row-split kernel) follow a T-token
    call to fp32 rounding, token by token."""
    import torch
    announce("chain through decode kernel")
    wl = W.Workload("chain_rows", 57, 4, 8, 2, 4, 128, 128, W.ACT_F32, 6, 0.05,
                    intermediates=True)
    inp = W.make_host_inputs(wl)
    pool_np = W.make_pool_host(wl)
    pool_multi = torch.from_numpy(pool_np).to(dev)
    out_multi, inter = run_gpu(inp, pool_multi, dev)
    pool_chain = torch.from_numpy(pool_np).to(dev)
    T = wl.tokens_per_seq
    for t in range(T):
        rows = np.arange(wl.num_seqs) * T + t
        step = W.HostInputs(wl.with_(tokens_per_seq=1, intermediates=False), inp.q[rows],
                            inp.k[rows], inp.v[rows], inp.a[rows], inp.b[rows], inp.A_log,
                            inp.dt_bias, inp.state_idx, None, np.ones(wl.num_seqs, np.int64), {})
        out_t, _ = run_gpu(step, pool_chain, dev)
        r = torch.from_numpy(rows).to(dev)
        assert rel_err(to_np(out_t), to_np(out_multi[r])) <= 1e-5, f"t={t}"
        slots = torch.from_numpy(inp.state_idx).long().to(dev)
        assert rel_err(pool_chain[slots].cpu().numpy(), inter[r].cpu().numpy()) <= 1e-5


def test_deterministic(dev):
    import torch
    announce("determinism")
    wl = W.VARLEN_LONG.with_(name="det", num_seqs=3, len_range=(20, 70), seed=51)
    inp = W.make_host_inputs(wl)
    pool_np = W.make_pool_host(wl)
    for family in (0, 1, 2):   # chunked under AUTO (mean length >= 32), column tiles, row split
        p1 = torch.from_numpy(pool_np).to(dev)
        p2 = torch.from_numpy(pool_np).to(dev)
        o1, _ = run_gpu(inp, p1, dev, kernel_family=family)
        o2, _ = run_gpu(inp, p2, dev, kernel_family=family)
        assert torch.equal(o1.nan_to_num(), o2.nan_to_num()) and torch.equal(p1, p2)


def test_strided_views_match_dense(dev):
    """q/k/v as column slices of one fused projection (token stride larger
    than the dense row, vLLM #37975 implementation: views of the fused
    projection) match the oracle, and give the dense result bit for bit."""
    import torch
    import linear_attention_recurrent_gating_amd as gdn
    announce("strided views")
    wl = W.Workload("strided", 52, 6, 3, 2, 4, 128, 128, W.ACT_BF16, 8, 0.05)
    inp = W.make_host_inputs(wl)
    d = W.to_torch(inp, dev)
    pool_np = W.make_pool_host(wl)
    p_dense = torch.from_numpy(pool_np).to(dev)
    o_dense, _ = run_gpu(inp, p_dense, dev, tensors=d)
    N = inp.num_tokens
    Hk, Hv, K, V = 2, 4, 128, 128
    width = 2 * Hk * K + Hv * V + 64           # padding keeps the stride a multiple of 8
    fused = torch.zeros(N, width, dtype=torch.bfloat16, device=dev)
    fused[:, :Hk * K] = d["q"].reshape(N, -1)
    fused[:, Hk * K:2 * Hk * K] = d["k"].reshape(N, -1)
    fused[:, 2 * Hk * K:2 * Hk * K + Hv * V] = d["v"].reshape(N, -1)
    q = fused[:, :Hk * K].view(N, Hk, K)
    k = fused[:, Hk * K:2 * Hk * K].view(N, Hk, K)
    v = fused[:, 2 * Hk * K:2 * Hk * K + Hv * V].view(N, Hv, V)
    assert q.stride(0) == width
    p_str = torch.from_numpy(pool_np).to(dev)
    out = torch.full((N, Hv, V), float("nan"), dtype=torch.bfloat16, device=dev)
    gdn.gdn_gating_delta_rule_update(q, k, v, d["a"], d["b"], d["A_log"], d["dt_bias"], p_str,
                                     d["state_idx"], None, out, tokens_per_seq=3)
    torch.cuda.synchronize()
    check_vs_oracle(inp, pool_np, p_str.cpu().numpy(), to_np(out), what="strided q/k/v")
    assert torch.equal(out, o_dense) and torch.equal(p_str, p_dense)


def test_no_final_writeback(dev):
    import torch
    import linear_attention_recurrent_gating_amd as gdn
    announce("no final writeback")
    wl = W.SPEC_VERIFY.with_(name="nfw", num_seqs=10, num_padded=2, num_slots=16, seed=53)
    inp = W.make_host_inputs(wl)
    pool_np = W.make_pool_host(wl)
    p1 = torch.from_numpy(pool_np).to(dev)
    o1, i1 = run_gpu(inp, p1, dev)
    p2 = torch.from_numpy(pool_np).to(dev)
    o2, i2 = run_gpu(inp, p2, dev, flags=gdn.GDN_FLAG_NO_FINAL_WRITEBACK)
    assert torch.equal(p2.cpu(), torch.from_numpy(pool_np)), "pool changed"
    assert torch.equal(o1.nan_to_num(), o2.nan_to_num()) and torch.equal(i1.nan_to_num(), i2.nan_to_num())


def test_debug_checks_reject_contract_violations(dev):
    import torch
    import linear_attention_recurrent_gating_amd as gdn
    announce("debug checks")
    wl = W.Workload("dbg", 54, 4, 1, 2, 4, 64, 64, W.ACT_F32, 6, 0.1)
    inp = W.make_host_inputs(wl)
    pool_np = W.make_pool_host(wl)
    pool = torch.from_numpy(pool_np).to(dev)
    d = W.to_torch(inp, dev)
    ok, _ = run_gpu(inp, pool.clone(), dev, tensors=d, flags=gdn.GDN_FLAG_DEBUG_CHECKS)
    dup = d["state_idx"].clone()
    dup[1] = dup[0]
    big = d["state_idx"].clone()
    big[2] = wl.num_slots
    for bad in (dup, big):
        dd = dict(d, state_idx=bad)
        with pytest.raises(gdn.GdnError) as ei:
            run_gpu(inp, pool, dev, tensors=dd, flags=gdn.GDN_FLAG_DEBUG_CHECKS)
        assert ei.value.status == 7
    assert torch.equal(pool.cpu(), torch.from_numpy(pool_np)), "a rejected call launched"
    wlv = W.Workload("dbgv", 55, 3, 1, 2, 4, 64, 64, W.ACT_F32, 6, 0.1, varlen=True,
                     len_range=(1, 3))
    inpv = W.make_host_inputs(wlv)
    dv = W.to_torch(inpv, dev)
    cu_bad = dv["cu_seqlens"].clone()
    cu_bad[1], cu_bad[2] = cu_bad[2], cu_bad[1]
    if cu_bad[1] != cu_bad[2]:
        with pytest.raises(gdn.GdnError):
            run_gpu(inpv, pool, dev, tensors=dict(dv, cu_seqlens=cu_bad),
                    flags=gdn.GDN_FLAG_DEBUG_CHECKS)


def test_empty_batch_launches_nothing(dev):
    import torch
    import linear_attention_recurrent_gating_amd as gdn
    z = torch.zeros(0, 2, 64, device=dev)
    zv = torch.zeros(0, 4, 64, device=dev)
    zab = torch.zeros(0, 4, device=dev)
    par = torch.zeros(4, device=dev)
    pool = torch.ones(3, 4, 64, 64, device=dev)
    idx = torch.zeros(0, dtype=torch.int32, device=dev)
    gdn.gdn_gating_delta_rule_update(z, z, zv, zab, zab, par, par, pool, idx, tokens_per_seq=1)
    torch.cuda.synchronize()
    assert torch.equal(pool, torch.ones_like(pool))


def test_side_stream(dev):
    """The call runs on the stream it is given."""
    import torch
    announce("side stream")
    wl = W.Workload("stream", 56, 4, 2, 2, 4, 128, 128, W.ACT_BF16, 6, 0.05)
    inp = W.make_host_inputs(wl)
    pool_np = W.make_pool_host(wl)
    p1 = torch.from_numpy(pool_np).to(dev)
    o1, _ = run_gpu(inp, p1, dev)
    p2 = torch.from_numpy(pool_np).to(dev)
    d = W.to_torch(inp, dev)
    s = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        o2, _ = run_gpu(inp, p2, dev, tensors=d, stream=s)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(p1, p2)


# ------------------------------------------------------------------ VK layout
@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_vk_small(dev, wl):
    full_check(wl, dev, layout="VK")


@pytest.mark.parametrize("K,V", ROW_SPLIT_PAIRS, ids=lambda x: str(x))
def test_vk_all_head_dims(dev, K, V):
    """The value-row kernel over every (K, V): one token and three tokens."""
    for act, seed, T in ((W.ACT_BF16, 70, 1), (W.ACT_F32, 71, 1), (W.ACT_BF16, 72, 3)):
        wl = W.Workload(f"vk_k{K}_v{V}_{act}_t{T}", seed + K + V, 5, T, 2, 4, K, V, act, 8, 0.05,
                        num_padded=1, intermediates=(T == 3))
        full_check(wl, dev, layout="VK")


@pytest.mark.parametrize("wl", [W.QWEN3NEXT_B64, W.SPEC_VERIFY, W.VARLEN_LONG,
                                W.SPEC_VERIFY.with_(name="spec_verify_weak_vk", decay="weak", seed=46)],
                         ids=lambda w: w.name)
def test_vk_workloads(dev, wl):
    """The value-row kernel on the named workloads (chosen explicitly: AUTO
    takes the chunked kernel for the long-varlen one)."""
    full_check(wl, dev, layout="VK", family=3)


@pytest.mark.parametrize("wl", [W.DECODE_B512, W.DECODE_B512_SHARD], ids=lambda w: w.name)
def test_vk_decode_b512_full_size(dev, wl):
    """The full-size decode with the VK pool (value-row kernel), every
    sequence against the oracle."""
    import torch
    import linear_attention_recurrent_gating_amd as gdn
    B = wl.num_seqs
    info = gdn.gdn_plan(gdn.make_config(torch.empty(B, wl.num_k_heads, 128),
                                        torch.empty(B, wl.num_v_heads, 128),
                                        torch.empty(1).expand(wl.num_slots, wl.num_v_heads,
                                                              128, 128),
                                        torch.zeros(B, dtype=torch.int32), state_layout="VK",
                                        tokens_per_seq=1), False)
    assert info.kernel_family == gdn.GDN_KERNEL_VALUE_ROWS
    check_full_size_decode(wl, dev, "VK")


def test_vk_chain_bitwise(dev):
    """With the VK layout the one-token and the multi-token calls run the same
    per-token code: T chained one-token calls equal one T-token call bit for
    bit, and each chained state equals the intermediate."""
    import torch
    announce("vk chain bitwise")
    wl = W.Workload("vk_chain", 73, 3, 6, 2, 4, 128, 128, W.ACT_BF16, 5, 0.05, intermediates=True)
    inp = W.make_host_inputs(wl)
    pool_np = to_layout(W.make_pool_host(wl), "VK")
    pool_multi = torch.from_numpy(pool_np).to(dev)
    out_multi, inter = run_gpu(inp, pool_multi, dev, layout="VK")
    pool_chain = torch.from_numpy(pool_np).to(dev)
    T = wl.tokens_per_seq
    for t in range(T):
        rows = np.arange(wl.num_seqs) * T + t
        step = W.HostInputs(wl.with_(tokens_per_seq=1, intermediates=False), inp.q[rows],
                            inp.k[rows], inp.v[rows], inp.a[rows], inp.b[rows], inp.A_log,
                            inp.dt_bias, inp.state_idx, None, np.ones(wl.num_seqs, np.int64),
                            {n: x[rows] for n, x in inp.bits.items()})
        out_t, _ = run_gpu(step, pool_chain, dev, layout="VK")
        r = torch.from_numpy(rows).to(dev)
        assert torch.equal(out_t, out_multi[r]), f"out differs at t={t}"
        for i in range(wl.num_seqs):
            assert torch.equal(pool_chain[int(inp.state_idx[i])], inter[int(rows[i])])
    assert torch.equal(pool_chain, pool_multi)


def test_vk_matches_kv(dev):
    """The two storage orders compute the same update (to fp32 rounding)."""
    import torch
    announce("vk vs kv")
    wl = W.Workload("vk_kv", 74, 8, 5, 2, 4, 128, 128, W.ACT_F32, 10, 0.05, intermediates=True)
    inp = W.make_host_inputs(wl)
    pool_np = W.make_pool_host(wl)
    p_kv = torch.from_numpy(pool_np).to(dev)
    p_vk = torch.from_numpy(to_layout(pool_np, "VK")).to(dev)
    o_kv, i_kv = run_gpu(inp, p_kv, dev)
    o_vk, i_vk = run_gpu(inp, p_vk, dev, layout="VK")
    assert rel_err(to_np(o_vk), to_np(o_kv)) <= 1e-5
    assert rel_err(p_vk.transpose(-1, -2).cpu().numpy(), p_kv.cpu().numpy()) <= 1e-5
    assert rel_err(i_vk.transpose(-1, -2).cpu().numpy(), i_kv.cpu().numpy()) <= 1e-5


def test_vk_waves_override(dev):
    import linear_attention_recurrent_gating_amd as gdn
    for waves in (4, 8):
        wl = W.Workload(f"vk_waves{waves}", 75, 4, 2, 2, 4, 128, 128, W.ACT_BF16, 6, 0.05)
        full_check(wl, dev, layout="VK", waves=waves, family=gdn.GDN_KERNEL_VALUE_ROWS)


# ------------------------------------------------- unfused pair, packed a/b
@pytest.mark.parametrize("act", [W.ACT_F32, W.ACT_BF16])
def test_gating_step_vs_oracle(dev, act):
    import torch
    import oracle
    import linear_attention_recurrent_gating_amd as gdn
    announce(f"gating step {act}")
    wl = W.Workload("gating", 80, 40, 3, 4, 8, 64, 64, act, 50, 0.05)
    inp = W.make_host_inputs(wl)
    d = W.to_torch(inp, dev)
    a2 = d["a"].view(inp.num_tokens, -1)
    g, beta = gdn.gdn_gating(a2, d["b"].view(inp.num_tokens, -1), d["A_log"], d["dt_bias"],
                             num_k_heads=wl.num_k_heads)
    torch.cuda.synchronize()
    g_ref, b_ref = oracle.gating(inp.a, inp.b, inp.A_log, inp.dt_bias)
    assert rel_err(np.exp(g.cpu().numpy().astype(np.float64)), np.exp(g_ref)) <= 1e-5
    assert rel_err(g.cpu().numpy(), g_ref) <= 1e-5
    assert rel_err(beta.cpu().numpy(), b_ref) <= 1e-5


UNFUSED_CASES = [
    ("KV", W.Workload("unf_decode", 81, 9, 1, 4, 8, 128, 128, W.ACT_BF16, 12, 0.05, num_padded=2)),
    ("KV", W.Workload("unf_spec", 82, 6, 1, 4, 8, 128, 128, W.ACT_BF16, 8, 0.05, varlen=True,
                      len_range=(1, 20), num_padded=1, intermediates=True)),
    ("VK", W.Workload("unf_decode_vk", 83, 9, 1, 4, 8, 128, 128, W.ACT_F32, 12, 0.05)),
    ("VK", W.Workload("unf_multi_vk", 84, 4, 5, 2, 4, 64, 128, W.ACT_BF16, 6, 0.05,
                      intermediates=True)),
]


@pytest.mark.parametrize("layout,wl", UNFUSED_CASES, ids=lambda x: x if isinstance(x, str) else x.name)
def test_unfused_pair_equals_fused(dev, layout, wl):
    """gdn_gating followed by gdn_recurrent_update (the per-token kernels on
    precomputed g and beta) matches the oracle, and gives the fused call's
    results bit for bit (gamma = exp of the same fp32 g)."""
    import torch
    import linear_attention_recurrent_gating_amd as gdn
    announce(f"unfused pair {wl.name} {layout}")
    inp = W.make_host_inputs(wl)
    d = W.to_torch(inp, dev)
    pool_np = to_layout(W.make_pool_host(wl), layout)
    p_fused = torch.from_numpy(pool_np).to(dev)
    o_fused, i_fused = run_gpu(inp, p_fused, dev, tensors=d, layout=layout)
    p_pair = torch.from_numpy(pool_np).to(dev)
    N = inp.num_tokens
    g, beta = gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"], num_k_heads=wl.num_k_heads)
    out = torch.full_like(o_fused, float("nan"))
    inter = None if i_fused is None else torch.full_like(i_fused, float("nan"))
    gdn.gdn_recurrent_update(d["q"], d["k"], d["v"], g, beta, p_pair, d["state_idx"],
                             d["cu_seqlens"], out, inter, tokens_per_seq=wl.tokens_per_seq,
                             state_layout=layout)
    torch.cuda.synchronize()
    check_vs_oracle(inp, pool_np, p_pair.cpu().numpy(), to_np(out),
                    None if inter is None else inter.cpu().numpy(), layout=layout,
                    what="unfused pair")
    assert torch.equal(out.nan_to_num(), o_fused.nan_to_num())
    assert torch.equal(p_pair, p_fused)
    if inter is not None:
        assert torch.equal(inter.nan_to_num(), i_fused.nan_to_num())
    assert N == g.shape[0]


@pytest.mark.parametrize("layout", ["KV", "VK"])
def test_packed_mixed_ba(dev, layout):
    """a and b read straight out of a projection packed per k-head as
    [N, H_k, 2G] (the G b-values, then the G a-values of the group; vLLM
    #37975 implementation) match the oracle on the dense a/b values, and give
    the dense result bit for bit, for the fused call and for the gating step."""
    import oracle
    import torch
    import linear_attention_recurrent_gating_amd as gdn
    announce(f"packed mixed_ba {layout}")
    wl = W.Workload("mixed_ba", 85, 7, 2, 4, 12, 64, 64, W.ACT_BF16, 9, 0.05)
    inp = W.make_host_inputs(wl)
    d = W.to_torch(inp, dev)
    pool_np = to_layout(W.make_pool_host(wl), layout)
    p_dense = torch.from_numpy(pool_np).to(dev)
    o_dense, _ = run_gpu(inp, p_dense, dev, tensors=d, layout=layout)
    N, Hk, G = inp.num_tokens, wl.num_k_heads, wl.group
    mixed = torch.empty(N, Hk, 2 * G, dtype=torch.bfloat16, device=dev)
    mixed[:, :, :G] = d["b"].view(N, Hk, G)
    mixed[:, :, G:] = d["a"].view(N, Hk, G)
    b_view, a_view = mixed[:, :, :G], mixed[:, :, G:]
    p_packed = torch.from_numpy(pool_np).to(dev)
    out = torch.full_like(o_dense, float("nan"))
    gdn.gdn_gating_delta_rule_update(d["q"], d["k"], d["v"], a_view, b_view, d["A_log"],
                                     d["dt_bias"], p_packed, d["state_idx"], None, out,
                                     tokens_per_seq=wl.tokens_per_seq, state_layout=layout)
    torch.cuda.synchronize()
    check_vs_oracle(inp, pool_np, p_packed.cpu().numpy(), to_np(out), layout=layout,
                    what="packed a/b")
    assert torch.equal(out, o_dense) and torch.equal(p_packed, p_dense)
    g1, b1 = gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"], num_k_heads=Hk)
    g2, b2 = gdn.gdn_gating(a_view, b_view, d["A_log"], d["dt_bias"])
    torch.cuda.synchronize()
    g_ref, b_ref = oracle.gating(inp.a, inp.b, inp.A_log, inp.dt_bias)
    assert rel_err(g2.cpu().numpy(), g_ref) <= 1e-5 and rel_err(b2.cpu().numpy(), b_ref) <= 1e-5
    assert torch.equal(g1, g2) and torch.equal(b1, b2)


# ------------------------------------------------------- bf16 state storage
def _bf16_within_one_ulp(got_bits, ref_bits):
    """True where two stored bf16 values differ by at most one bf16 ulp (of
    the larger magnitude), or by no more than the fp32 arithmetic noise
    (1e-5 of the largest reference magnitude) for elements near zero, where
    a tiny value's ulp is smaller than that noise."""
    g = _bits_to_f32(got_bits).astype(np.float64)
    r = _bits_to_f32(ref_bits).astype(np.float64)
    mag = np.maximum(np.abs(g), np.abs(r))
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-38))) - 7)
    return np.abs(g - r) <= np.maximum(ulp, 1e-5 * float(np.max(np.abs(r))))


def _bits_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


STATE_BF16_CASES = [
    ("KV", W.Workload("bf16state_decode", 90, 9, 1, 4, 8, 128, 128, W.ACT_BF16, 12, 0.05,
                      num_padded=2)),
    ("KV", W.Workload("bf16state_spec", 91, 6, 1, 4, 8, 128, 128, W.ACT_BF16, 8, 0.05,
                      varlen=True, len_range=(1, 20), num_padded=1, intermediates=True)),
    ("KV", W.Workload("bf16state_rows_f32", 92, 5, 3, 2, 4, 64, 64, W.ACT_F32, 8, 0.05,
                      intermediates=True)),
    ("KV:cols", W.Workload("bf16state_cols_f32", 97, 5, 3, 2, 4, 64, 64, W.ACT_F32, 8, 0.05,
                           intermediates=True)),
    ("KV:cols", W.Workload("bf16state_cols_spec", 98, 6, 1, 4, 8, 128, 128, W.ACT_BF16, 8, 0.05,
                           varlen=True, len_range=(1, 20), num_padded=1, intermediates=True)),
    ("VK", W.Workload("bf16state_vk_decode", 93, 9, 1, 4, 8, 128, 128, W.ACT_BF16, 12, 0.05)),
    ("VK", W.Workload("bf16state_vk_multi", 94, 4, 5, 2, 4, 64, 128, W.ACT_BF16, 6, 0.05,
                      intermediates=True)),
    ("KV", W.QWEN3NEXT_B64.with_(name="bf16state_qwen3next_b64", seed=95)),
    ("KV:rows", W.Workload("bf16state_rows_spec", 96, 6, 1, 4, 8, 128, 128, W.ACT_BF16, 8, 0.05,
                           varlen=True, len_range=(1, 20), num_padded=1, intermediates=True)),
]


@pytest.mark.parametrize("layout,wl", STATE_BF16_CASES,
                         ids=lambda x: x if isinstance(x, str) else x.name)
def test_bf16_state_storage(dev, layout, wl):
    """State stored as bf16 (fp32 arithmetic): outputs to the activation
    bar, stored states within one bf16 ulp of the oracle's single rounding,
    untouched slots and padded rows bit-identical."""
    import torch
    announce(f"bf16 state {wl.name} {layout}")
    layout, _, kind = layout.partition(":")
    family = {"rows": 2, "cols": 1}.get(kind, 0)   # GDN_KERNEL_ROW_SPLIT / _COLUMN_TILES
    inp = W.make_host_inputs(wl)
    bits, _ = W.round_to_bf16(to_layout(W.make_pool_host(wl), layout))
    pool = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    out, inter = run_gpu(inp, pool, dev, layout=layout, kernel_family=family)
    seqs = np.arange(wl.num_seqs)
    o_ref, s_ref, i_ref, _ = oracle_on_seqs(inp, bits[np.maximum(inp.state_idx, 0)], seqs,
                                            intermediates=wl.intermediates, layout=layout)
    live, dead = live_rows(inp)
    out_np = to_np(out)
    assert rel_err(out_np[live], o_ref[live]) <= tol_for(wl)
    assert np.all(np.isnan(out_np[dead]))
    after = pool.view(torch.int16).cpu().numpy().view(np.uint16)
    lv = inp.state_idx >= 0
    got = after[inp.state_idx[lv]]
    assert np.all(_bf16_within_one_ulp(got, s_ref[lv])), "final state beyond one bf16 ulp"
    assert rel_err(_bits_to_f32(got), _bits_to_f32(s_ref[lv])) <= 2e-2
    assert np.mean(got == s_ref[lv]) > 0.99, "most stored elements should round identically"
    untouched = np.setdiff1d(np.arange(wl.num_slots), inp.state_idx[lv])
    assert np.array_equal(after[untouched], bits[untouched])
    if wl.intermediates:
        ib = inter.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.all(_bf16_within_one_ulp(ib[live], i_ref[live]))
        assert np.all(ib[dead] == 0x7FC0), "padded rows of bf16 intermediates were written"
