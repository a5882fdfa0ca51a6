"""Seeded synthetic workloads for the GDN decode state update.

This module only draws and lays out inputs; it holds none of the update's
arithmetic, so both the HIP path and the CPU oracle can be fed from it.

The shapes follow the serving workloads the pages discuss: the fused
gating + recurrent update kernel of vLLM PR #35777 (implementation section:
inputs A_log, a, b, dt_bias plus q/k/v and the recurrent state) and the
sglang PR #18271 profile (Benchmarking and Profiling: bs=512 on a TP4 shard,
grid [1, 4, 4k], which fixes 8 v-heads per shard and V = 128).  Head counts
use the Qwen3-Next layout (16 k-heads, 32 v-heads, K = V = 128); GQA groups
consecutive v-heads under one k-head (vLLM PR #37975, implementation section:
the a/b projection is reshaped per k-head into 2*H_v/H_k values).

Draw order for one workload, from ``numpy.random.default_rng(seed)``:
  lengths (varlen only), q, k, v, a, b, dt_bias, A_log, slot permutation,
  padding positions.  The state pool comes from its own generator (seed+1),
  on the device it will live on.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

ACT_F32 = "f32"
ACT_BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    num_seqs: int            # B
    tokens_per_seq: int      # T (fixed-length mode); ignored when varlen
    num_k_heads: int         # H_k
    num_v_heads: int         # H_v
    head_k_dim: int          # K
    head_v_dim: int          # V
    act: str                 # activation dtype of q, k, v, a, b, out
    num_slots: int           # rows in the state pool
    pool_std: float          # std-dev of the initial fp32 state
    varlen: bool = False     # pass cu_seqlens
    len_range: tuple = (1, 1)  # inclusive U{lo..hi} lengths when varlen
    num_padded: int = 0      # sequences whose slot index is -1
    intermediates: bool = False
    fixed_slots: Optional[tuple] = None  # explicit slot indices (tiny case)
    decay: str = "normal"    # "normal": A_log = log U[1,16]; "weak": log U[1e-3,1e-2]

    @property
    def group(self) -> int:
        return self.num_v_heads // self.num_k_heads

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the decode path.
TINY_F32 = Workload("tiny_fp32_b2", 0, 2, 1, 2, 4, 32, 32, ACT_F32, 4, 0.1,
                    fixed_slots=(2, 0))
QWEN3NEXT_B64 = Workload("qwen3next_decode_b64", 1, 64, 1, 16, 32, 128, 128,
                         ACT_BF16, 1024, 0.05)
DECODE_B512 = Workload("decode_b512_hk16_hv32", 2, 512, 1, 16, 32, 128, 128,
                       ACT_BF16, 4096, 0.05)
DECODE_B512_SHARD = Workload("decode_b512_hk4_hv8", 3, 512, 1, 4, 8, 128, 128,
                             ACT_BF16, 4096, 0.05)
SPEC_VERIFY = Workload("spec_verify_b128_t4", 4, 128, 4, 16, 32, 128, 128,
                       ACT_BF16, 1024, 0.05, varlen=True, len_range=(4, 4),
                       num_padded=13, intermediates=True)
VARLEN_LONG = Workload("varlen_long_8x64_2048", 5, 8, 1, 16, 32, 128, 128,
                       ACT_BF16, 64, 0.05, varlen=True, len_range=(64, 2048))

ALL = {w.name: w for w in (TINY_F32, QWEN3NEXT_B64, DECODE_B512,
                           DECODE_B512_SHARD, SPEC_VERIFY, VARLEN_LONG)}


def round_to_bf16(x: np.ndarray):
    """fp32 -> bf16 by round-to-nearest-even; returns (bits uint16, fp32 values)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    vals = (r.astype(np.uint32) << 16).view(np.float32)
    return r, vals


@dataclasses.dataclass
class HostInputs:
    """Host copies of one workload's inputs (all but the state pool)."""
    wl: Workload
    q: np.ndarray        # [N, H_k, K] fp32 values (bf16-representable if act is bf16)
    k: np.ndarray        # [N, H_k, K]
    v: np.ndarray        # [N, H_v, V]
    a: np.ndarray        # [N, H_v]
    b: np.ndarray        # [N, H_v]
    A_log: np.ndarray    # [H_v] fp32
    dt_bias: np.ndarray  # [H_v] fp32
    state_idx: np.ndarray  # [B] int32, -1 = padding
    cu_seqlens: Optional[np.ndarray]  # [B+1] int32 or None
    lengths: np.ndarray  # [B] tokens per sequence
    bits: dict           # name -> uint16 bf16 bits (bf16 workloads only)

    @property
    def num_tokens(self) -> int:
        return int(self.lengths.sum())


def make_host_inputs(wl: Workload) -> HostInputs:
    rng = np.random.default_rng(wl.seed)
    B = wl.num_seqs
    if wl.varlen:
        lo, hi = wl.len_range
        lengths = rng.integers(lo, hi + 1, size=B).astype(np.int64)
    else:
        lengths = np.full(B, wl.tokens_per_seq, dtype=np.int64)
    N = int(lengths.sum())
    f32 = np.float32
    q = rng.standard_normal((N, wl.num_k_heads, wl.head_k_dim), dtype=f32)
    k = rng.standard_normal((N, wl.num_k_heads, wl.head_k_dim), dtype=f32)
    v = rng.standard_normal((N, wl.num_v_heads, wl.head_v_dim), dtype=f32)
    a = rng.standard_normal((N, wl.num_v_heads), dtype=f32)
    b = rng.standard_normal((N, wl.num_v_heads), dtype=f32)
    dt_bias = (rng.standard_normal(wl.num_v_heads, dtype=f32) * f32(0.5)).astype(f32)
    if wl.decay == "weak":
        A_log = np.log(rng.uniform(1e-3, 1e-2, size=wl.num_v_heads)).astype(f32)
    else:
        A_log = np.log(rng.uniform(1.0, 16.0, size=wl.num_v_heads)).astype(f32)
    if wl.fixed_slots is not None:
        idx = np.asarray(wl.fixed_slots, dtype=np.int32)
    else:
        idx = rng.permutation(wl.num_slots)[:B].astype(np.int32)
    if wl.num_padded:
        pad = rng.choice(B, size=wl.num_padded, replace=False)
        idx[pad] = -1
    cu = None
    if wl.varlen:
        cu = np.zeros(B + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
    acts = {"q": q, "k": k, "v": v, "a": a, "b": b}
    bits = {}
    if wl.act == ACT_BF16:
        for name, arr in list(acts.items()):
            bits[name], acts[name] = round_to_bf16(arr)
    return HostInputs(wl, acts["q"], acts["k"], acts["v"], acts["a"], acts["b"],
                      A_log, dt_bias, idx, cu, lengths, bits)


def pool_shape(wl: Workload):
    return (wl.num_slots, wl.num_v_heads, wl.head_k_dim, wl.head_v_dim)


def make_pool_host(wl: Workload) -> np.ndarray:
    """Initial fp32 state pool drawn on the host (small workloads)."""
    rng = np.random.default_rng(wl.seed + 1)
    return (rng.standard_normal(pool_shape(wl), dtype=np.float32)
            * np.float32(wl.pool_std)).astype(np.float32)


def make_pool_torch(wl: Workload, device):
    """Initial fp32 state pool drawn directly on ``device`` with a seeded torch
    generator (large workloads: the pool is GiBs)."""
    import torch
    dev = torch.device(device)
    if dev.type == "cpu":
        return torch.from_numpy(make_pool_host(wl))
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed + 1)
    pool = torch.randn(pool_shape(wl), generator=g, device=dev, dtype=torch.float32)
    pool.mul_(wl.pool_std)
    return pool


def to_torch(inp: HostInputs, device):
    """Device tensors for the HIP path: activations in the workload's dtype."""
    import torch
    dev = torch.device(device)
    out = {}
    for name in ("q", "k", "v", "a", "b"):
        if inp.wl.act == ACT_BF16:
            t = torch.from_numpy(inp.bits[name].view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(getattr(inp, name))
        out[name] = t.to(dev).contiguous()
    out["A_log"] = torch.from_numpy(inp.A_log).to(dev)
    out["dt_bias"] = torch.from_numpy(inp.dt_bias).to(dev)
    out["state_idx"] = torch.from_numpy(inp.state_idx).to(dev)
    out["cu_seqlens"] = (torch.from_numpy(inp.cu_seqlens).to(dev)
                         if inp.cu_seqlens is not None else None)
    return out


def active_updates(inp: HostInputs) -> int:
    """(sequence, v-head, token) steps of non-padded sequences."""
    live = inp.state_idx >= 0
    return int(inp.lengths[live].sum()) * inp.wl.num_v_heads


def algorithmic_bytes(inp: HostInputs, final_writeback: bool = True, state_bytes: int = 4) -> int:
    """Bytes the update must move: state read + (intermediates) + final write of
    every live (sequence, v-head), plus every token's activations and the
    per-call parameters.  Re-reads of shared q/k are not counted.
    state_bytes: 4 for an fp32 state pool, 2 for bf16 storage."""
    wl = inp.wl
    e = 2 if wl.act == ACT_BF16 else 4
    K, V, Hk, Hv = wl.head_k_dim, wl.head_v_dim, wl.num_k_heads, wl.num_v_heads
    tile = K * V * state_bytes
    live = inp.state_idx >= 0
    nlive = int(live.sum())
    state = nlive * Hv * tile * (1 + (1 if final_writeback else 0))
    if wl.intermediates:
        state += int(inp.lengths[live].sum()) * Hv * tile
    ntok = int(inp.lengths[live].sum())
    act = ntok * (2 * Hk * K * e + 2 * Hv * V * e + 2 * Hv * e)
    params = 8 * Hv + 4 * wl.num_seqs + (4 * (wl.num_seqs + 1) if wl.varlen else 0)
    return state + act + params


FLOPS_PER_ELEMENT = 7   # per state element and token: decay 1, S^T k 2, k u^T 2, S^T q 2


def recurrent_flops(inp: HostInputs) -> int:
    """Flops of the token-by-token update for every live (sequence, v-head,
    token): 7 per state element (the decay, the two reductions and the rank-1
    update).  The gates and the q/k norms add O(K + V) per token and are not
    counted."""
    wl = inp.wl
    return active_updates(inp) * wl.head_k_dim * wl.head_v_dim * FLOPS_PER_ELEMENT


CHUNK_TOKENS = 64  # tokens per chunk of the chunked forward


def chunked_flops(inp: HostInputs, chunk: int = CHUNK_TOKENS) -> int:
    """Flops of the dense products of the chunked (WY) form for every live
    (sequence, v-head): per chunk of L tokens, the key-key and query-key
    products (2 x 2 L^2 K), the products with the chunk-start state (2 x 2 L K V),
    the triangular factor times R and the masked query-key matrix times U
    (2 x 2 L^2 V), the state update (2 L K V) and the triangular inverse
    (L^3 / 3 multiply-adds)."""
    wl = inp.wl
    K, V = wl.head_k_dim, wl.head_v_dim
    total = 0
    for L, s in zip(inp.lengths, inp.state_idx):
        if s < 0:
            continue
        full, tail = divmod(int(L), chunk)
        for n, c in ((full, chunk), (1 if tail else 0, tail)):
            total += n * (4 * c * c * K + 4 * c * c * V + 6 * c * K * V + (2 * c ** 3) // 3)
    return total * wl.num_v_heads
