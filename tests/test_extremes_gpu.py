"""Saturated gates and degenerate vectors against the oracle: a + dt_bias far
into both tails (softplus linear or vanishing, decay exp(g) underflowing to
zero), b far into both tails (beta = 0 or 1), A_log from tiny to large,
all-zero q or k rows (the eps inside the root keeps them finite), and
single-token spikes of strong decay in the middle of a sequence."""
import numpy as np
import pytest

from gpu_helpers import (TOL_STATE_GUARD, announce, live_rows, oracle_on_seqs, rel_err, run_gpu,
                         to_np, tol_for)
from linear_attention_recurrent_gating_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


def _extreme_inputs(wl, seed):
    inp = W.make_host_inputs(wl)
    rng = np.random.default_rng(seed)
    N, Hv, Hk = inp.num_tokens, wl.num_v_heads, wl.num_k_heads
    f32 = np.float32
    tails = np.array([-60.0, -12.0, 0.0, 12.0, 60.0], f32)
    inp.a = np.where(rng.random((N, Hv)) < 0.4, rng.choice(tails, (N, Hv)), inp.a).astype(f32)
    inp.b = np.where(rng.random((N, Hv)) < 0.4, rng.choice(tails, (N, Hv)), inp.b).astype(f32)
    inp.A_log = np.log(np.array([1e-3, 1.0, 16.0, 40.0][:Hv] + [2.0] * max(0, Hv - 4), f32))
    # zero q or k rows
    for arr in (inp.q, inp.k):
        rows = rng.choice(N, size=max(1, N // 8), replace=False)
        heads = rng.integers(0, Hk, size=rows.size)
        arr[rows, heads] = 0.0
    # strong-decay spikes: a token whose gate input is large, amid ordinary ones
    spikes = rng.choice(N, size=max(1, N // 16), replace=False)
    inp.a[spikes] = 8.0
    if wl.act == W.ACT_BF16:   # the edited values are bf16-exact; refresh the bit patterns
        for name in ("q", "k", "a", "b"):
            inp.bits[name], arr = W.round_to_bf16(getattr(inp, name))
            setattr(inp, name, arr)
    return inp


CASES = [
    ("row_split", W.Workload("ext_rows", 180, 5, 12, 2, 4, 64, 64, W.ACT_F32, 8, 0.05,
                             intermediates=True), 2),
    ("column_tiles", W.Workload("ext_cols", 181, 5, 12, 2, 4, 64, 64, W.ACT_F32, 8, 0.05,
                                intermediates=True), 1),
    ("decode", W.Workload("ext_dec", 182, 40, 1, 2, 4, 128, 128, W.ACT_F32, 48, 0.05), 0),
    ("chunked", W.Workload("ext_chunk", 183, 4, 1, 2, 4, 128, 128, W.ACT_F32, 6, 0.05,
                           varlen=True, len_range=(50, 160)), 4),
    ("row_split_bf16", W.Workload("ext_rows16", 184, 5, 12, 2, 4, 128, 128, W.ACT_BF16, 8, 0.05,
                                  intermediates=True), 2),
    ("chunked_bf16", W.Workload("ext_chunk16", 185, 4, 1, 2, 4, 128, 128, W.ACT_BF16, 6, 0.05,
                                varlen=True, len_range=(50, 160)), 4),
]


@pytest.mark.parametrize("name,wl,family", CASES, ids=[c[0] for c in CASES])
def test_extreme_gates_and_zero_vectors(dev, name, wl, family):
    import torch
    announce(f"extremes {name}")
    inp = _extreme_inputs(wl, wl.seed)
    pool_np = W.make_pool_host(wl)
    pool = torch.from_numpy(pool_np).to(dev)
    out, inter = run_gpu(inp, pool, dev, kernel_family=family)
    o_ref, s_ref, i_ref, _ = oracle_on_seqs(inp, pool_np[np.maximum(inp.state_idx, 0)],
                                            np.arange(wl.num_seqs), intermediates=wl.intermediates)
    live, _ = live_rows(inp)
    out_np = to_np(out)
    assert np.all(np.isfinite(out_np[live])), "non-finite outputs"
    assert rel_err(out_np[live], o_ref[live]) <= tol_for(wl), "out"
    lv = inp.state_idx >= 0
    after = pool.cpu().numpy()
    assert np.all(np.isfinite(after)), "non-finite states"
    assert rel_err(after[inp.state_idx[lv]], s_ref[lv]) <= TOL_STATE_GUARD, "state"
    if wl.intermediates:
        assert rel_err(inter.cpu().numpy()[live], i_ref[live]) <= TOL_STATE_GUARD, "inter"


LONG = [
    ("row_split", 2), ("column_tiles", 1), ("chunked", 4),
]


@pytest.mark.parametrize("name,family", LONG, ids=[c[0] for c in LONG])
def test_long_sequences_fp32(dev, name, family):
    """Sequences of 3000 to 8192 tokens with fp32 activations (and a weakly
    decaying head, whose state carries far): rounding does not accumulate
    past the fp32 bar."""
    import torch
    announce(f"long fp32 {name}")
    wl = W.Workload(f"long_{name}", 190, 2, 1, 1, 2, 128, 128, W.ACT_F32, 3, 0.05, varlen=True,
                    len_range=(3000, 8192), decay="weak")
    inp = W.make_host_inputs(wl)
    pool_np = W.make_pool_host(wl)
    pool = torch.from_numpy(pool_np).to(dev)
    out, _ = run_gpu(inp, pool, dev, kernel_family=family)
    o_ref, s_ref, _, _ = oracle_on_seqs(inp, pool_np[np.maximum(inp.state_idx, 0)],
                                        np.arange(wl.num_seqs))
    assert rel_err(to_np(out), o_ref) <= tol_for(wl), "out"
    assert rel_err(pool.cpu().numpy()[inp.state_idx], s_ref) <= TOL_STATE_GUARD, "state"
