"""The chunked forward (64-token chunks on the matrix cores) against the CPU
oracle.  The chunked form is the same operation as the token-by-token
update, so the oracle is the per-token recurrence itself: outputs and final
states must agree within the activation dtype's tolerance.  Cases span one
and several chunks, ragged tails, chunk-size boundaries, GQA, both layouts,
bf16 state storage, padding and empty sequences."""
import numpy as np
import pytest

from gpu_helpers import (TOL_STATE_GUARD, announce, check_vs_oracle, live_rows, oracle_on_seqs,
                         rel_err, to_layout, to_np, tol_for)
from linear_attention_recurrent_gating_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


FORMS = ["one_kernel", "workspace"]


def make_workspace(d, pool, inp, fill=0xFF):
    """The two-kernel form's workspace, pre-filled with a byte pattern (0xFF:
    NaN floats and bf16s), so that nothing can rely on it starting clean."""
    import linear_attention_recurrent_gating_amd as gdn
    ws = gdn.chunk_workspace(d["q"], d["v"], pool, d["state_idx"], d["cu_seqlens"],
                             tokens_per_seq=inp.wl.tokens_per_seq)
    ws.fill_(fill)
    return ws


def run_chunked(inp, pool, dev, layout="KV", flags=0, pregated=False, form="one_kernel",
                ws_fill=0xFF):
    """One call of gdn_chunk_gated_delta_rule_fwd (form "one_kernel": no
    workspace; "workspace": the prep + state-pass kernels over a workspace),
    or of gdn_recurrent_update with the chunked family on precomputed gates.
    Output rows that must not be written are pre-filled with NaN."""
    import torch
    import linear_attention_recurrent_gating_amd as gdn
    wl = inp.wl
    d = W.to_torch(inp, dev)
    act = torch.bfloat16 if wl.act == W.ACT_BF16 else torch.float32
    out = torch.full((inp.num_tokens, wl.num_v_heads, wl.head_v_dim), float("nan"), dtype=act,
                     device=dev)
    if pregated:
        g, beta = gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"],
                                 num_k_heads=wl.num_k_heads)
        gdn.gdn_recurrent_update(d["q"], d["k"], d["v"], g, beta, pool, d["state_idx"],
                                 d["cu_seqlens"], out, tokens_per_seq=wl.tokens_per_seq,
                                 flags=flags, kernel_family=gdn.GDN_KERNEL_CHUNKED,
                                 state_layout=layout)
    else:
        ws = make_workspace(d, pool, inp, ws_fill) if form == "workspace" else None
        gdn.gdn_chunk_gated_delta_rule_fwd(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"],
                                           d["dt_bias"], pool, d["state_idx"], d["cu_seqlens"], out,
                                           workspace=ws, tokens_per_seq=wl.tokens_per_seq,
                                           flags=flags, state_layout=layout)
    torch.cuda.synchronize()
    return out


def check_chunked(wl, dev, layout="KV", state_dtype="f32", flags=0, pregated=False,
                  state_tol=TOL_STATE_GUARD, form="one_kernel"):
    """Whole-batch parity of the chunked forward: out rows of live sequences,
    final states, untouched slots and rows."""
    import torch
    import linear_attention_recurrent_gating_amd as gdn
    announce(f"chunked {wl.name} B={wl.num_seqs} H={wl.num_k_heads}/{wl.num_v_heads} "
             f"K={wl.head_k_dim} V={wl.head_v_dim} act={wl.act} layout={layout} "
             f"state={state_dtype} flags={flags} pregated={pregated} form={form}")
    inp = W.make_host_inputs(wl)
    pool_f32 = to_layout(W.make_pool_host(wl), layout)
    if state_dtype == "bf16":
        pool_np, _ = W.round_to_bf16(pool_f32)
        pool = torch.from_numpy(pool_np.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        pool_np = pool_f32
        pool = torch.from_numpy(pool_np).to(dev)
    out = run_chunked(inp, pool, dev, layout=layout, flags=flags, pregated=pregated, form=form)
    seqs = np.arange(wl.num_seqs)
    o_ref, s_ref, _, _ = oracle_on_seqs(inp, pool_np[np.maximum(inp.state_idx, 0)], seqs,
                                        no_final_writeback=bool(flags & gdn.GDN_FLAG_NO_FINAL_WRITEBACK),
                                        layout=layout)
    live, dead = live_rows(inp)
    out_np = to_np(out)
    e_out = rel_err(out_np[live], o_ref[live])
    tol = tol_for(wl)
    assert e_out <= tol, f"out error {e_out:.3e} > {tol}"
    assert np.all(np.isnan(out_np[dead])), "padded sequences wrote outputs"
    if state_dtype == "bf16":
        pool_after = pool.view(torch.int16).cpu().numpy().view(np.uint16)
        as_f32 = lambda bits: (bits.astype(np.uint32) << 16).view(np.float32)
    else:
        pool_after = pool.cpu().numpy()
        as_f32 = lambda x: x
    lv = inp.state_idx >= 0
    e_state = 0.0
    if not (flags & gdn.GDN_FLAG_NO_FINAL_WRITEBACK):
        e_state = rel_err(as_f32(pool_after[inp.state_idx[lv]]), as_f32(s_ref[lv]))
        assert e_state <= min(tol, state_tol), f"state error {e_state:.3e}"
        untouched = np.setdiff1d(np.arange(wl.num_slots), inp.state_idx[lv])
    else:
        untouched = np.arange(wl.num_slots)
    assert np.array_equal(pool_after[untouched], pool_np[untouched]), "untouched slots changed"
    print(f"{wl.name}: out {e_out:.2e} state {e_state:.2e}")
    return e_out, e_state


CASES = [
    # several chunks with a ragged tail, and lengths 0..1 (no chunk / one token)
    W.Workload("ck_k128v128_bf16_varlen", 70, 5, 1, 2, 4, 128, 128, W.ACT_BF16, 8, 0.05,
               varlen=True, len_range=(0, 300)),
    W.Workload("ck_k128v128_f32_varlen", 71, 4, 1, 2, 4, 128, 128, W.ACT_F32, 6, 0.05,
               varlen=True, len_range=(1, 260)),
    # fixed length, no cu_seqlens: two full chunks and a two-token tail
    W.Workload("ck_k64v64_f32_t130", 72, 3, 130, 2, 4, 64, 64, W.ACT_F32, 5, 0.1),
    W.Workload("ck_k32v32_f32_pad", 73, 6, 1, 2, 4, 32, 32, W.ACT_F32, 9, 0.1, varlen=True,
               len_range=(0, 150), num_padded=2),
    W.Workload("ck_k64v128_g4_bf16", 74, 3, 1, 1, 4, 64, 128, W.ACT_BF16, 4, 0.05, varlen=True,
               len_range=(60, 200)),
    W.Workload("ck_k128v64_bf16", 75, 3, 1, 2, 4, 128, 64, W.ACT_BF16, 4, 0.05, varlen=True,
               len_range=(64, 192)),
    W.Workload("ck_k32v128_g3_f32", 76, 3, 1, 2, 6, 32, 128, W.ACT_F32, 4, 0.05, varlen=True,
               len_range=(1, 140)),
    W.Workload("ck_k128v32_bf16", 77, 3, 1, 2, 4, 128, 32, W.ACT_BF16, 4, 0.05, varlen=True,
               len_range=(1, 140)),
    W.Workload("ck_weak_decay_f32", 78, 3, 1, 2, 4, 128, 128, W.ACT_F32, 4, 0.05, varlen=True,
               len_range=(100, 400), decay="weak"),
    W.Workload("ck_weak_decay_bf16", 79, 4, 1, 2, 4, 128, 128, W.ACT_BF16, 5, 0.05, varlen=True,
               len_range=(100, 400), decay="weak"),
]


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_chunked_small(dev, wl, form):
    check_chunked(wl, dev, form=form)


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("T", [63, 64, 65, 128])
def test_chunked_chunk_boundaries(dev, T, form):
    wl = W.Workload(f"ck_t{T}", 80 + T, 2, T, 2, 4, 128, 128, W.ACT_F32, 4, 0.05)
    check_chunked(wl, dev, form=form)


@pytest.mark.parametrize("form", FORMS)
def test_chunked_varlen_long(dev, form):
    """The long-varlen workload (8 sequences of 64..2048 tokens) at full size."""
    check_chunked(W.VARLEN_LONG, dev, form=form)


@pytest.mark.parametrize("form", FORMS)
def test_chunked_varlen_long_weak_decay(dev, form):
    check_chunked(W.VARLEN_LONG.with_(name="varlen_long_weak_ck", decay="weak", seed=45), dev,
                  form=form)


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("layout,state", [("VK", "f32"), ("KV", "bf16"), ("VK", "bf16")])
def test_chunked_layouts_and_bf16_state(dev, layout, state, form):
    wl = W.Workload(f"ck_{layout}_{state}", 90, 4, 1, 2, 4, 128, 128, W.ACT_BF16, 6, 0.05,
                    varlen=True, len_range=(1, 200), num_padded=1)
    # bf16 storage: the final state is rounded once (half an ulp, 2^-9)
    check_chunked(wl, dev, layout=layout, state_dtype=state,
                  state_tol=TOL_STATE_GUARD if state == "f32" else 2 ** -8, form=form)


def test_chunked_many_short_sequences(dev):
    """Many sequences of 0..70 tokens (most under one chunk, several empty):
    every sequence starts a new chunk slot, and most slots of the workspace
    belong to no chunk."""
    wl = W.Workload("ck_many_short", 98, 40, 1, 2, 4, 64, 128, W.ACT_BF16, 48, 0.05, varlen=True,
                    len_range=(0, 70), num_padded=5)
    check_chunked(wl, dev, form="workspace")


def test_chunked_workspace_contents_do_not_matter(dev):
    """The two-kernel form reads only workspace bytes its first kernel wrote:
    a workspace pre-filled with NaN patterns and one pre-filled with zeros
    give the same results bit for bit, and match the one-kernel form to fp32
    rounding."""
    import torch
    announce("chunked workspace contents")
    wl = W.Workload("ck_ws_fill", 99, 5, 1, 2, 4, 128, 128, W.ACT_F32, 7, 0.05, varlen=True,
                    len_range=(1, 200), num_padded=1)
    inp = W.make_host_inputs(wl)
    pool_np = W.make_pool_host(wl)
    outs, pools = [], []
    for fill in (0xFF, 0x00):
        p = torch.from_numpy(pool_np).to(dev)
        outs.append(run_chunked(inp, p, dev, form="workspace", ws_fill=fill))
        pools.append(p)
    assert torch.equal(outs[0].nan_to_num(), outs[1].nan_to_num()) and torch.equal(pools[0], pools[1])
    p1 = torch.from_numpy(pool_np).to(dev)
    o1 = run_chunked(inp, p1, dev, form="one_kernel")
    assert rel_err(to_np(outs[0]).reshape(-1)[~np.isnan(to_np(o1).reshape(-1))],
                   to_np(o1).reshape(-1)[~np.isnan(to_np(o1).reshape(-1))]) <= 1e-4
    assert rel_err(pools[0].cpu().numpy(), p1.cpu().numpy()) <= 1e-4


def test_chunked_pregated(dev):
    wl = W.Workload("ck_pregated", 91, 3, 1, 2, 4, 128, 128, W.ACT_BF16, 4, 0.05, varlen=True,
                    len_range=(30, 150))
    check_chunked(wl, dev, pregated=True)


@pytest.mark.parametrize("form", FORMS)
def test_chunked_no_final_writeback(dev, form):
    import linear_attention_recurrent_gating_amd as gdn
    wl = W.Workload("ck_nowb", 92, 3, 1, 2, 4, 64, 64, W.ACT_F32, 4, 0.05, varlen=True,
                    len_range=(10, 100))
    check_chunked(wl, dev, flags=gdn.GDN_FLAG_NO_FINAL_WRITEBACK, form=form)


@pytest.mark.parametrize("form", FORMS)
def test_chunked_deterministic(dev, form):
    import torch
    announce(f"chunked determinism {form}")
    wl = W.Workload("ck_det", 93, 3, 1, 2, 4, 128, 128, W.ACT_BF16, 4, 0.05, varlen=True,
                    len_range=(50, 200))
    inp = W.make_host_inputs(wl)
    pool_np = W.make_pool_host(wl)
    p1 = torch.from_numpy(pool_np).to(dev)
    p2 = torch.from_numpy(pool_np).to(dev)
    o1 = run_chunked(inp, p1, dev, form=form)
    o2 = run_chunked(inp, p2, dev, form=form)
    assert torch.equal(o1.nan_to_num(), o2.nan_to_num()) and torch.equal(p1, p2)


@pytest.mark.parametrize("form", FORMS)
def test_chunked_matches_recurrent_kernel(dev, form):
    """The chunked and the per-token kernels agree to fp32 rounding on fp32
    activations (both against each other, not only against the oracle)."""
    import torch
    import linear_attention_recurrent_gating_amd as gdn
    announce(f"chunked vs recurrent {form}")
    wl = W.Workload("ck_vs_rec", 94, 4, 1, 2, 4, 128, 128, W.ACT_F32, 5, 0.05, varlen=True,
                    len_range=(100, 300))
    inp = W.make_host_inputs(wl)
    pool_np = W.make_pool_host(wl)
    p_ck = torch.from_numpy(pool_np).to(dev)
    p_rec = torch.from_numpy(pool_np).to(dev)
    o_ck = run_chunked(inp, p_ck, dev, form=form)
    d = W.to_torch(inp, dev)
    o_rec = gdn.gdn_gating_delta_rule_update(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"],
                                             d["dt_bias"], p_rec, d["state_idx"], d["cu_seqlens"])
    torch.cuda.synchronize()
    assert rel_err(to_np(o_ck), to_np(o_rec)) <= 1e-4
    assert rel_err(p_ck.cpu().numpy(), p_rec.cpu().numpy()) <= 1e-4


@pytest.mark.parametrize("form", FORMS)
def test_chunked_all_padded(dev, form):
    """Every sequence padded: nothing is read or written."""
    import torch
    announce(f"chunked all padded {form}")
    wl = W.Workload("ck_all_pad", 96, 3, 1, 2, 4, 64, 64, W.ACT_BF16, 6, 0.05, varlen=True,
                    len_range=(5, 70), num_padded=3)
    inp = W.make_host_inputs(wl)
    pool = torch.from_numpy(W.make_pool_host(wl)).to(dev)
    pool0 = pool.clone()
    out = run_chunked(inp, pool, dev, form=form)
    assert torch.isnan(out).all() and torch.equal(pool, pool0)


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("layout", ["KV", "VK"])
def test_chunked_strided_and_packed_inputs(dev, layout, form):
    """q/k/v as column slices of one fused projection and a/b packed per
    k-head ([N, H_k, 2G]: the G b-values, then the G a-values; vLLM #37975
    implementation) match the oracle, and give the dense chunked result bit
    for bit."""
    import torch
    import linear_attention_recurrent_gating_amd as gdn
    announce(f"chunked strided/packed {layout}")
    wl = W.Workload("ck_strided", 97, 3, 100, 2, 6, 128, 64, W.ACT_BF16, 5, 0.05)
    inp = W.make_host_inputs(wl)
    d = W.to_torch(inp, dev)
    pool_np = to_layout(W.make_pool_host(wl), layout)
    p_dense = torch.from_numpy(pool_np).to(dev)
    o_dense = run_chunked(inp, p_dense, dev, layout=layout, form=form)
    N, Hk, Hv, K, V, G = inp.num_tokens, 2, 6, 128, 64, 3
    width = 2 * Hk * K + Hv * V + 40           # the stride stays a multiple of 8
    fused = torch.zeros(N, width, dtype=torch.bfloat16, device=dev)
    fused[:, :Hk * K] = d["q"].reshape(N, -1)
    fused[:, Hk * K:2 * Hk * K] = d["k"].reshape(N, -1)
    fused[:, 2 * Hk * K:2 * Hk * K + Hv * V] = d["v"].reshape(N, -1)
    q = fused[:, :Hk * K].view(N, Hk, K)
    k = fused[:, Hk * K:2 * Hk * K].view(N, Hk, K)
    v = fused[:, 2 * Hk * K:2 * Hk * K + Hv * V].view(N, Hv, V)
    mixed = torch.empty(N, Hk, 2 * G, dtype=torch.bfloat16, device=dev)
    mixed[:, :, :G] = d["b"].view(N, Hk, G)
    mixed[:, :, G:] = d["a"].view(N, Hk, G)
    p_str = torch.from_numpy(pool_np).to(dev)
    out = torch.full_like(o_dense, float("nan"))
    ws = make_workspace(d, p_str, inp) if form == "workspace" else None
    gdn.gdn_chunk_gated_delta_rule_fwd(q, k, v, mixed[:, :, G:], mixed[:, :, :G], d["A_log"],
                                       d["dt_bias"], p_str, d["state_idx"], None, out,
                                       workspace=ws, tokens_per_seq=wl.tokens_per_seq,
                                       state_layout=layout)
    torch.cuda.synchronize()
    check_vs_oracle(inp, pool_np, p_str.cpu().numpy(), to_np(out), layout=layout,
                    what="chunked strided/packed")
    assert torch.equal(out, o_dense) and torch.equal(p_str, p_dense)
