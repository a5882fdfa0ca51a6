"""Wide and odd GQA ratios (G = H_v / H_k of 5, 6, 8 and 16) through every
kernel family: the v-heads of one k-head share its staged q/k, and the
workgroup shapes change with G (heads per workgroup are a divisor of G within
the wavefront and LDS limits).  Outputs, final states and intermediates match
the oracle; padded and untouched slots keep their bytes."""
import numpy as np
import pytest

from gpu_helpers import (TOL_STATE_GUARD, announce, live_rows, oracle_on_seqs, rel_err, run_gpu,
                         to_layout, to_np, tol_for)
from linear_attention_recurrent_gating_amd import workloads as W

pytestmark = pytest.mark.gpu


def _wl(name, seed, B, T, Hk, Hv, K, V, act, **kw):
    return W.Workload(name, seed, B, T, Hk, Hv, K, V, act, B + 3, 0.05, **kw)


# (id, workload, kernel family, layout, tiling overrides)
CASES = [
    ("g5_rows_decode", _wl("gqa5_dec", 140, 6, 1, 2, 10, 128, 128, W.ACT_BF16, num_padded=1),
     2, "KV", {}),
    ("g8_auto_decode_k64", _wl("gqa8_dec64", 141, 5, 1, 1, 8, 64, 64, W.ACT_F32), 0, "KV", {}),
    ("g16_rows_token_loop", _wl("gqa16_spec", 142, 5, 1, 1, 16, 128, 128, W.ACT_BF16, varlen=True,
                                len_range=(1, 6), num_padded=1, intermediates=True), 2, "KV", {}),
    ("g6_rows_32_rows_per_lane", _wl("gqa6_rpl32", 143, 5, 1, 1, 6, 128, 128, W.ACT_BF16),
     2, "KV", {"block_k": 64, "waves_per_group": 6}),
    ("g6_rows_token_loop_32", _wl("gqa6_tl32", 144, 4, 3, 1, 6, 128, 128, W.ACT_BF16,
                                  intermediates=True), 2, "KV", {"block_k": 64, "waves_per_group": 6}),
    ("g16_column_tiles", _wl("gqa16_cols", 145, 4, 3, 2, 32, 128, 64, W.ACT_BF16), 1, "KV", {}),
    ("g5_column_tiles_f32", _wl("gqa5_cols", 146, 4, 2, 1, 5, 64, 128, W.ACT_F32,
                                intermediates=True), 1, "KV", {"block_v": 32}),
    ("g8_value_rows", _wl("gqa8_vk", 147, 4, 2, 2, 16, 128, 128, W.ACT_BF16, num_padded=1),
     3, "VK", {}),
    ("g16_chunked", _wl("gqa16_chunk", 148, 3, 1, 1, 16, 128, 128, W.ACT_BF16, varlen=True,
                        len_range=(20, 150)), 4, "KV", {}),
    ("g5_chunked_vk", _wl("gqa5_chunk_vk", 149, 3, 1, 2, 10, 64, 64, W.ACT_F32, varlen=True,
                          len_range=(30, 100)), 4, "VK", {}),
]


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


@pytest.mark.parametrize("name,wl,family,layout,over", CASES, ids=[c[0] for c in CASES])
def test_gqa_ratio(dev, name, wl, family, layout, over):
    import torch
    announce(f"gqa {name}: H {wl.num_k_heads}/{wl.num_v_heads} K={wl.head_k_dim} "
             f"V={wl.head_v_dim} family {family} {layout} {over}")
    inp = W.make_host_inputs(wl)
    pool_np = to_layout(W.make_pool_host(wl), layout)
    pool = torch.from_numpy(pool_np).to(dev)
    out, inter = run_gpu(inp, pool, dev, kernel_family=family, layout=layout, **over)
    o_ref, s_ref, i_ref, _ = oracle_on_seqs(inp, pool_np[np.maximum(inp.state_idx, 0)],
                                            np.arange(wl.num_seqs),
                                            intermediates=wl.intermediates, layout=layout)
    live, dead = live_rows(inp)
    out_np = to_np(out)
    assert rel_err(out_np[live], o_ref[live]) <= tol_for(wl), "out"
    assert np.all(np.isnan(out_np[dead])), "padded sequences wrote outputs"
    after = pool.cpu().numpy()
    lv = inp.state_idx >= 0
    assert rel_err(after[inp.state_idx[lv]], s_ref[lv]) <= min(tol_for(wl), TOL_STATE_GUARD), "state"
    untouched = np.setdiff1d(np.arange(wl.num_slots), inp.state_idx[lv])
    assert np.array_equal(after[untouched], pool_np[untouched]), "untouched slots changed"
    if wl.intermediates:
        inter_np = inter.cpu().numpy()
        assert rel_err(inter_np[live], i_ref[live]) <= min(tol_for(wl), TOL_STATE_GUARD), "inter"
        assert np.all(np.isnan(inter_np[dead])), "padded sequences wrote intermediates"
