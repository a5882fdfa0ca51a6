"""HIP graph capture of the entry points (torch.cuda.graph): a captured call,
replayed several times with the program's own eager work (restoring the
state pool, clearing the outputs) and synchronisations between replays, gives
the eager call's results bit for bit on every replay.  The library enqueues
kernels only -- no allocation, memset or host synchronisation -- so a serving
loop can capture it."""
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


REPLAYS = 3

CASES = [
    ("decode_row_split", W.Workload("graph_decode", 120, 16, 1, 4, 8, 128, 128, W.ACT_BF16, 40, 0.05,
                                    num_padded=2), 0),
    ("spec_token_loop", W.Workload("graph_spec", 121, 12, 1, 4, 8, 128, 128, W.ACT_BF16, 30, 0.05,
                                   varlen=True, len_range=(1, 6), num_padded=1,
                                   intermediates=True), 0),
    ("column_tiles", W.Workload("graph_cols", 122, 6, 5, 2, 4, 64, 128, W.ACT_F32, 12, 0.05,
                                intermediates=True), 1),
    ("chunked", W.Workload("graph_chunked", 123, 4, 1, 2, 4, 128, 128, W.ACT_BF16, 8, 0.05,
                           varlen=True, len_range=(40, 200)), 4),
    ("value_rows", W.Workload("graph_vk", 124, 8, 3, 2, 4, 128, 64, W.ACT_BF16, 16, 0.05), -1),
]


def _call(gdn, d, wl, pool, out, inter, family):
    layout = gdn.GDN_LAYOUT_VK if family < 0 else gdn.GDN_LAYOUT_KV
    gdn.gdn_gating_delta_rule_update(
        d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], pool, d["state_idx"],
        d["cu_seqlens"], out, inter, tokens_per_seq=wl.tokens_per_seq,
        kernel_family=max(family, 0), state_layout=layout)


@pytest.mark.parametrize("name,wl,family", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(dev, name, wl, family):
    import torch
    import linear_attention_recurrent_gating_amd as gdn
    announce(f"graph capture {name}")
    inp = W.make_host_inputs(wl)
    d = W.to_torch(inp, dev)
    pool_np = W.make_pool_host(wl)
    if family < 0:
        pool_np = np.ascontiguousarray(np.swapaxes(pool_np, -1, -2))
    pool0 = torch.from_numpy(pool_np).to(dev)
    act = torch.bfloat16 if wl.act == W.ACT_BF16 else torch.float32
    N = inp.num_tokens

    def buffers():
        out = torch.full((N, wl.num_v_heads, wl.head_v_dim), float("nan"), dtype=act, device=dev)
        inter = None
        if wl.intermediates:
            inter = torch.full((N, wl.num_v_heads) + tuple(pool0.shape[2:]), float("nan"),
                               dtype=pool0.dtype, device=dev)
        return out, inter

    pool_e = pool0.clone()
    out_e, inter_e = buffers()
    _call(gdn, d, wl, pool_e, out_e, inter_e, family)
    torch.cuda.synchronize()

    pool_g = pool0.clone()
    out_g, inter_g = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):     # warm-up on a side stream, as capture requires
        _call(gdn, d, wl, pool_g.clone(), out_g.clone(), None if inter_g is None else inter_g.clone(),
              family)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _call(gdn, d, wl, pool_g, out_g, inter_g, family)
    torch.cuda.synchronize()
    assert torch.equal(pool_g, pool0), "capture must not execute the kernels"

    for rep in range(REPLAYS):
        pool_g.copy_(pool0)
        out_g.fill_(float("nan"))
        if inter_g is not None:
            inter_g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.nan_to_num(), out_e.nan_to_num()), f"out differs on replay {rep}"
        assert torch.equal(pool_g, pool_e), f"state differs on replay {rep}"
        if inter_g is not None:
            assert torch.equal(inter_g.nan_to_num(), inter_e.nan_to_num()), \
                f"intermediates differ on replay {rep}"


def test_graph_unfused_pair(dev):
    """The unfused pair (gating kernel, then the update from g and beta)
    captured as two nodes of one graph."""
    import torch
    import linear_attention_recurrent_gating_amd as gdn
    announce("graph capture unfused pair")
    wl = W.Workload("graph_pair", 125, 10, 1, 4, 8, 128, 128, W.ACT_BF16, 24, 0.05, num_padded=1)
    inp = W.make_host_inputs(wl)
    d = W.to_torch(inp, dev)
    pool0 = torch.from_numpy(W.make_pool_host(wl)).to(dev)
    N = inp.num_tokens
    g = torch.empty(N, wl.num_v_heads, dtype=torch.float32, device=dev)
    beta = torch.empty_like(g)

    def pair(pool, out):
        gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"], g, beta,
                       num_k_heads=wl.num_k_heads)
        gdn.gdn_recurrent_update(d["q"], d["k"], d["v"], g, beta, pool, d["state_idx"], None, out,
                                 tokens_per_seq=1)

    pool_e = pool0.clone()
    out_e = torch.full((N, wl.num_v_heads, wl.head_v_dim), float("nan"), dtype=torch.bfloat16,
                       device=dev)
    pair(pool_e, out_e)
    torch.cuda.synchronize()
    pool_g = pool0.clone()
    out_g = torch.full_like(out_e, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pair(pool_g.clone(), out_g.clone())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pair(pool_g, out_g)
    for rep in range(REPLAYS):
        pool_g.copy_(pool0)
        out_g.fill_(float("nan"))
        g.zero_()
        beta.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.nan_to_num(), out_e.nan_to_num()), f"out differs on replay {rep}"
        assert torch.equal(pool_g, pool_e), f"state differs on replay {rep}"
