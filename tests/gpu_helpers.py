"""Shared helpers of the GPU parity tests: run the HIP path and the oracle on
the same seeded inputs and compare them."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from linear_attention_recurrent_gating_amd import workloads as W

# Tolerances on max|x - ref| / max|ref|, per compared tensor.
TOL_F32 = 1e-4      # fp32 activations
TOL_BF16 = 2e-2     # bf16 q/k/v/a/b with fp32 state
# Guard on the fp32 state with bf16 activations: the kernel widens the same
# bf16 values the oracle gets, so only fp32 arithmetic separates the states;
# a wrong state carry would show far above this.
TOL_STATE_GUARD = 1e-4


def announce(msg: str):
    """Names the case on the real stderr (not captured) before GPU work."""
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def rel_err(x, ref) -> float:
    """max|x - ref| / max|ref|, in float64, taken in blocks of leading-axis
    rows so that full-size states (a GiB of fp32) need little extra memory."""
    x = np.asarray(x)
    ref = np.asarray(ref)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if x.size == 0:
        return 0.0
    rows = x.reshape(x.shape[0], -1) if x.ndim > 1 else x.reshape(-1, 1)
    rrows = ref.reshape(rows.shape)
    step = max(1, (1 << 22) // max(1, rows.shape[1]))
    err = scale = 0.0
    for i in range(0, rows.shape[0], step):
        xb = rows[i:i + step].astype(np.float64)
        rb = rrows[i:i + step].astype(np.float64)
        e = float(np.max(np.abs(xb - rb)))
        if not np.isfinite(e):
            return float("inf")
        err = max(err, e)
        scale = max(scale, float(np.max(np.abs(rb))))
    return err / scale if scale > 0 else err


def tol_for(wl) -> float:
    return TOL_BF16 if wl.act == W.ACT_BF16 else TOL_F32


def to_np(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def live_rows(inp):
    """Token rows of live (non-padded) sequences, and of padded ones."""
    starts = np.concatenate([[0], np.cumsum(inp.lengths)[:-1]]).astype(np.int64)
    live, dead = [], []
    for i, (s, L) in enumerate(zip(starts, inp.lengths)):
        (live if inp.state_idx[i] >= 0 else dead).append(np.arange(s, s + L))
    cat = lambda xs: np.concatenate(xs) if xs else np.zeros(0, np.int64)
    return cat(live), cat(dead)


def to_layout(pool_kv: np.ndarray, layout: str) -> np.ndarray:
    """A [slots, H_v, K, V] pool (or one tile stack) in the given storage order."""
    if layout == "KV":
        return pool_kv
    return np.ascontiguousarray(np.swapaxes(pool_kv, -1, -2))


def run_gpu(inp, pool, device, intermediates=None, flags=0, block_v=0, waves_per_group=0,
            tensors=None, stream=None, kernel_family=0, block_k=0, layout="KV"):
    """One call of the HIP path.  Returns (out, inter) as torch tensors; rows
    that must not be written are pre-filled with NaN."""
    import torch
    import linear_attention_recurrent_gating_amd as gdn
    wl = inp.wl
    d = tensors if tensors is not None else W.to_torch(inp, device)
    if intermediates is None:
        intermediates = wl.intermediates
    act = torch.bfloat16 if wl.act == W.ACT_BF16 else torch.float32
    N = inp.num_tokens
    out = torch.full((N, wl.num_v_heads, wl.head_v_dim), float("nan"), dtype=act, device=device)
    inter = None
    if intermediates:
        tile = (wl.head_k_dim, wl.head_v_dim) if layout == "KV" else (wl.head_v_dim, wl.head_k_dim)
        inter = torch.full((N, wl.num_v_heads) + tile, float("nan"), dtype=pool.dtype,
                           device=device)
    gdn.gdn_gating_delta_rule_update(
        d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], pool, d["state_idx"],
        d["cu_seqlens"], out, inter, tokens_per_seq=wl.tokens_per_seq, flags=flags,
        kernel_family=kernel_family, block_v=block_v, block_k=block_k,
        waves_per_group=waves_per_group, stream=stream, state_layout=layout)
    torch.cuda.synchronize()
    return out, inter


def sub_inputs(inp, seqs):
    """The sub-batch of sequences `seqs` (with their token rows), re-slotted to
    0..len(seqs)-1, for the oracle."""
    starts = np.concatenate([[0], np.cumsum(inp.lengths)[:-1]]).astype(np.int64)
    rows = np.concatenate([np.arange(starts[i], starts[i] + inp.lengths[i]) for i in seqs]) \
        if len(seqs) else np.zeros(0, np.int64)
    lengths = inp.lengths[seqs]
    cu = np.zeros(len(seqs) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    idx = np.where(inp.state_idx[seqs] >= 0, np.arange(len(seqs)), -1).astype(np.int32)
    return dict(q=inp.q[rows], k=inp.k[rows], v=inp.v[rows], a=inp.a[rows], b=inp.b[rows],
                A_log=inp.A_log, dt_bias=inp.dt_bias, state_idx=idx, cu_seqlens=cu), rows


def oracle_on_seqs(inp, pool0_rows, seqs, intermediates=False, no_final_writeback=False,
                   layout="KV"):
    """Oracle on the sequences `seqs`; pool0_rows [len(seqs), H_v, K, V] (or
    [.., V, K] for layout "VK") holds their initial states.  Returns (out rows,
    final states, inter rows, rows) in that layout."""
    d, rows = sub_inputs(inp, seqs)
    pool = np.ascontiguousarray(pool0_rows).copy()   # float32, or uint16 bf16 bit patterns
    assert pool.dtype in (np.float32, np.uint16)
    out, inter = oracle.update(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                               pool, d["state_idx"], d["cu_seqlens"], intermediates=intermediates,
                               no_final_writeback=no_final_writeback, state_layout=layout)
    return out, pool, inter, rows


def check_vs_oracle(inp, pool0_np, pool_after_np, out_np, inter_np=None, layout="KV",
                    prefilled=True, what=""):
    """One call's fp32-state results against the oracle on the same inputs:
    out rows of live sequences within the activation tolerance; final states
    and intermediates within it and within the fp32 state guard; the last
    intermediate of each sequence equal to its final state bit for bit;
    untouched pool slots unchanged; and, where out and intermediates were
    pre-filled with NaN, padded rows left unwritten.  pool0_np / pool_after_np
    are the whole pool before and after the call."""
    wl = inp.wl
    seqs = np.arange(wl.num_seqs)
    o_ref, s_ref, i_ref, _ = oracle_on_seqs(inp, pool0_np[np.maximum(inp.state_idx, 0)], seqs,
                                            intermediates=inter_np is not None, layout=layout)
    tol = tol_for(wl)
    live, dead = live_rows(inp)
    e_out = rel_err(out_np[live], o_ref[live])
    assert e_out <= tol, f"{what}: out error {e_out:.3e} > {tol}"
    lv = inp.state_idx >= 0
    e_state = rel_err(pool_after_np[inp.state_idx[lv]], s_ref[lv])
    assert e_state <= min(tol, TOL_STATE_GUARD), f"{what}: state error {e_state:.3e}"
    untouched = np.setdiff1d(np.arange(pool0_np.shape[0]), inp.state_idx[lv])
    assert np.array_equal(pool_after_np[untouched], pool0_np[untouched]), \
        f"{what}: untouched slots changed"
    if prefilled:
        assert np.all(np.isnan(out_np[dead])), f"{what}: padded sequences wrote outputs"
    if inter_np is not None:
        e_inter = rel_err(inter_np[live], i_ref[live])
        assert e_inter <= min(tol, TOL_STATE_GUARD), f"{what}: intermediate error {e_inter:.3e}"
        if prefilled:
            assert np.all(np.isnan(inter_np[dead])), f"{what}: padded rows of intermediates written"
        ends = np.cumsum(inp.lengths) - 1
        for i in np.nonzero(lv & (inp.lengths > 0))[0]:
            assert np.array_equal(inter_np[ends[i]], pool_after_np[inp.state_idx[i]]), \
                f"{what}: last intermediate of sequence {i} is not its final state"
    return e_out, e_state
