"""The Python binding's fast paths on the GPU: the stream handle it derives
without building a torch stream object, and PreparedUpdate (tensors bound
once) against the plain call, bit for bit, across in-place changes of the
inputs and slot indices and on a side stream."""
import numpy as np
import pytest

from gpu_helpers import announce
from linear_attention_recurrent_gating_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


def test_stream_handle_is_torch_current_stream(dev):
    import torch
    import linear_attention_recurrent_gating_amd as gdn
    announce("stream handle")
    assert gdn._stream_handle(None, dev) == torch.cuda.current_stream(dev).cuda_stream
    side = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(side):
        assert gdn._stream_handle(None, dev) == side.cuda_stream
    assert gdn._stream_handle(side, dev) == side.cuda_stream
    assert gdn._stream_handle(side.cuda_stream, dev) == side.cuda_stream


CASES = [
    W.Workload("prep_decode", 160, 6, 1, 4, 8, 128, 128, W.ACT_BF16, 12, 0.05, num_padded=1),
    W.Workload("prep_spec", 161, 5, 1, 2, 4, 64, 128, W.ACT_F32, 10, 0.05, varlen=True,
               len_range=(1, 5), num_padded=1, intermediates=True),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_prepared_update_matches_call(dev, wl):
    import torch
    import linear_attention_recurrent_gating_amd as gdn
    announce(f"prepared update {wl.name}")
    inp = W.make_host_inputs(wl)
    d = W.to_torch(inp, dev)
    pool0 = torch.from_numpy(W.make_pool_host(wl)).to(dev)
    N = inp.num_tokens
    act = torch.bfloat16 if wl.act == W.ACT_BF16 else torch.float32

    def buffers():
        out = torch.full((N, wl.num_v_heads, wl.head_v_dim), float("nan"), dtype=act, device=dev)
        inter = None
        if wl.intermediates:
            inter = torch.full((N, wl.num_v_heads, wl.head_k_dim, wl.head_v_dim), float("nan"),
                               device=dev)
        return out, inter

    pool_c, pool_p = pool0.clone(), pool0.clone()
    out_c, inter_c = buffers()
    out_p, inter_p = buffers()
    args = (d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"])
    prep = gdn.PreparedUpdate(*args, pool_p, d["state_idx"], d["cu_seqlens"], out_p, inter_p,
                              tokens_per_seq=wl.tokens_per_seq)
    side = torch.cuda.Stream(device=dev)
    rng = np.random.default_rng(wl.seed)
    for rep in range(3):
        if rep > 0:   # new contents, same storage: inputs and slot assignment
            d["q"].copy_(torch.randn_like(d["q"], dtype=torch.float32).to(act))
            live = inp.state_idx >= 0
            perm = inp.state_idx.copy()
            perm[live] = rng.permutation(wl.num_slots)[:int(live.sum())]
            d["state_idx"].copy_(torch.from_numpy(perm))
        gdn.gdn_gating_delta_rule_update(*args, pool_c, d["state_idx"], d["cu_seqlens"], out_c,
                                         inter_c, tokens_per_seq=wl.tokens_per_seq)
        if rep == 2:
            side.wait_stream(torch.cuda.current_stream(dev))
            assert prep(side) is out_p
            torch.cuda.current_stream(dev).wait_stream(side)
        else:
            assert prep() is out_p
        torch.cuda.synchronize()
        assert torch.equal(out_c.nan_to_num(), out_p.nan_to_num()), f"out, call {rep}"
        assert torch.equal(pool_c, pool_p), f"pool, call {rep}"
        if inter_c is not None:
            assert torch.equal(inter_c.nan_to_num(), inter_p.nan_to_num()), f"inter, call {rep}"


def test_prepared_update_rejects_bad_arguments(dev):
    import torch
    import linear_attention_recurrent_gating_amd as gdn
    announce("prepared update errors")
    wl = CASES[0]
    d = W.to_torch(W.make_host_inputs(wl), dev)
    pool = torch.zeros(W.pool_shape(wl), device=dev)
    with pytest.raises(gdn.GdnError):   # an unsupported tile override, caught at construction
        gdn.PreparedUpdate(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], pool,
                           d["state_idx"], None, block_v=24)
