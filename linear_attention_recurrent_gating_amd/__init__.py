"""Python binding of libgdn: the fused sigmoid-gating + gated delta-rule state
update (Gated DeltaNet decode) on AMD MI355X.

Argument marshalling only.  Every step of the update runs in the HIP kernels
of ``_lib/libgdn.so`` behind the C-ABI declared in ``include/gdn.h``; PyTorch
supplies device memory and the stream.  The library is loaded on first use,
and every entry point raises ImportError when it has not been built
(``python -m linear_attention_recurrent_gating_amd.build``); there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
# GDN_LIBRARY names another build of the same sources (the tests load a
# build whose host code is compiled with AddressSanitizer this way).
LIB_PATH = os.environ.get("GDN_LIBRARY") or os.path.join(_PKG, "_lib", "libgdn.so")

GDN_OK = 0
GDN_DTYPE_F32 = 0
GDN_DTYPE_BF16 = 1
GDN_FLAG_NO_FINAL_WRITEBACK = 0x1
GDN_FLAG_DEBUG_CHECKS = 0x2
GDN_KERNEL_AUTO = 0
GDN_KERNEL_COLUMN_TILES = 1
GDN_KERNEL_ROW_SPLIT = 2
GDN_KERNEL_VALUE_ROWS = 3
GDN_KERNEL_CHUNKED = 4
GDN_LAYOUT_KV = 0
GDN_LAYOUT_VK = 1
_LAYOUTS = {"KV": GDN_LAYOUT_KV, "VK": GDN_LAYOUT_VK, GDN_LAYOUT_KV: GDN_LAYOUT_KV,
            GDN_LAYOUT_VK: GDN_LAYOUT_VK}

STATUS_NAMES = {0: "GDN_OK", 1: "GDN_ERR_NULL_POINTER", 2: "GDN_ERR_BAD_SHAPE",
                3: "GDN_ERR_UNSUPPORTED_SHAPE", 4: "GDN_ERR_UNSUPPORTED_DTYPE",
                5: "GDN_ERR_MISALIGNED", 6: "GDN_ERR_LAUNCH", 7: "GDN_ERR_BAD_ARGUMENT"}

# Every symbol include/gdn.h declares.
EXPORTED = ("gdn_default_config", "gdn_gating_delta_rule_update", "gdn_gating",
            "gdn_recurrent_update", "gdn_chunk_gated_delta_rule_fwd", "gdn_chunk_workspace_bytes",
            "gdn_chunk_gated_delta_rule_fwd_noalloc",
            "gdn_validate", "gdn_plan", "gdn_status_string",
            "gdn_last_error_message", "gdn_abi_version")


class GdnConfig(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("tokens_per_seq", ctypes.c_int32),
                ("num_tokens", ctypes.c_int64), ("num_k_heads", ctypes.c_int32),
                ("num_v_heads", ctypes.c_int32), ("head_k_dim", ctypes.c_int32),
                ("head_v_dim", ctypes.c_int32), ("num_slots", ctypes.c_int64),
                ("act_dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("l2norm_eps", ctypes.c_float), ("q_stride_tok", ctypes.c_int64),
                ("k_stride_tok", ctypes.c_int64), ("v_stride_tok", ctypes.c_int64),
                ("ab_stride_tok", ctypes.c_int64), ("ab_stride_khead", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("state_layout", ctypes.c_int32),
                ("state_dtype", ctypes.c_int32),
                ("kernel_family", ctypes.c_int32),
                ("block_v", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("waves_per_group", ctypes.c_int32)]


class GdnLaunchInfo(ctypes.Structure):
    _fields_ = [("kernel_family", ctypes.c_int32), ("block_v", ctypes.c_int32),
                ("block_k", ctypes.c_int32), ("waves_per_group", ctypes.c_int32),
                ("tokens_per_chunk", ctypes.c_int32), ("multi_token", ctypes.c_int32),
                ("workgroups", ctypes.c_int64), ("threads_per_group", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32)]


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libgdn is not built ({LIB_PATH} missing): run "
                          "`python -m linear_attention_recurrent_gating_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, C = ctypes.c_void_p, ctypes.POINTER(GdnConfig)
    lib.gdn_default_config.argtypes = [C]
    lib.gdn_default_config.restype = None
    lib.gdn_gating_delta_rule_update.argtypes = [P] * 12 + [C, P]
    lib.gdn_gating_delta_rule_update.restype = ctypes.c_int
    lib.gdn_gating.argtypes = [P] * 6 + [C, P]
    lib.gdn_gating.restype = ctypes.c_int
    lib.gdn_recurrent_update.argtypes = [P] * 10 + [C, P]
    lib.gdn_recurrent_update.restype = ctypes.c_int
    lib.gdn_chunk_gated_delta_rule_fwd.argtypes = [P] * 12 + [ctypes.c_size_t, C, P]
    lib.gdn_chunk_gated_delta_rule_fwd.restype = ctypes.c_int
    lib.gdn_chunk_workspace_bytes.argtypes = [C]
    lib.gdn_chunk_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_chunk_gated_delta_rule_fwd_noalloc.argtypes = [P] * 11 + [C, P]
    lib.gdn_chunk_gated_delta_rule_fwd_noalloc.restype = ctypes.c_int
    lib.gdn_validate.argtypes = [P] * 12 + [C]
    lib.gdn_validate.restype = ctypes.c_int
    lib.gdn_plan.argtypes = [C, ctypes.c_int, ctypes.c_int, ctypes.POINTER(GdnLaunchInfo)]
    lib.gdn_plan.restype = ctypes.c_int
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_last_error_message.argtypes = []
    lib.gdn_last_error_message.restype = ctypes.c_char_p
    lib.gdn_abi_version.argtypes = []
    lib.gdn_abi_version.restype = ctypes.c_int
    return lib


_LIB_HANDLE: Optional[ctypes.CDLL] = None


def raw_library() -> ctypes.CDLL:
    """The loaded C library (loaded on first use)."""
    global _LIB_HANDLE
    if _LIB_HANDLE is None:
        _LIB_HANDLE = _load()
    return _LIB_HANDLE


def gdn_abi_version() -> int:
    return raw_library().gdn_abi_version()


def gdn_status_string(status: int) -> str:
    return raw_library().gdn_status_string(status).decode()


def gdn_last_error_message() -> str:
    return raw_library().gdn_last_error_message().decode()


def gdn_default_config() -> GdnConfig:
    cfg = GdnConfig()
    raw_library().gdn_default_config(ctypes.byref(cfg))
    return cfg


def _check(status: int):
    if status != GDN_OK:
        raise GdnError(status, gdn_last_error_message() or gdn_status_string(status))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(stream, device) -> int:
    """The hipStream_t to enqueue on: ``stream`` (a torch stream or a raw
    handle), else torch's current stream on ``device``."""
    if stream is None:
        import torch
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:   # same handle as current_stream().cuda_stream, without the object
            return raw(device.index if device.index is not None else torch.cuda.current_device())
        return torch.cuda.current_stream(device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _ab_strides(a, b, N, Hv, Hk):
    """(ab_stride_tok, ab_stride_khead) of a/b given as dense [N, H_v] tensors or
    as [N, H_k, G] views (e.g. slices of a projection packed per k-head)."""
    G = Hv // Hk
    if a.shape != b.shape:
        raise ValueError("a and b must have the same shape")
    if a.dim() not in (2, 3):
        raise ValueError("a/b must be [N, H_v] or [N, H_k, G]")
    if N == 0:   # nothing is read: any strides do
        if tuple(a.shape) not in ((0, Hv), (0, Hk, G)):
            raise ValueError(f"a/b must be [0, {Hv}] or [0, {Hk}, {G}]")
        return 0, 0
    if a.stride() != b.stride():
        raise ValueError("a and b must have the same strides")
    if a.dim() == 2:
        if tuple(a.shape) != (N, Hv) or (Hv > 1 and a.stride(1) != 1):
            raise ValueError(f"a/b must be [{N}, {Hv}] with unit stride over heads")
        return (a.stride(0) if N > 1 else 0), 0
    if tuple(a.shape) != (N, Hk, G) or (G > 1 and a.stride(2) != 1):
        raise ValueError(f"a/b views must be [{N}, {Hk}, {G}] with unit innermost stride")
    return (a.stride(0) if N > 1 else 0), (a.stride(1) if Hk > 1 else G)


def _check_tensors(q, k, v, a, b, A_log, dt_bias, state_pool, state_idx, cu_seqlens, out,
                   intermediate_states, state_layout=GDN_LAYOUT_KV):
    """dtype/shape/device/layout checks the C-ABI cannot make on raw pointers."""
    import torch
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[0] != q.shape[0]:
        raise ValueError("q, k must be [N, H_k, K] and v [N, H_v, V] with the same N")
    N, Hv, V = v.shape
    K = q.shape[2]
    act = q.dtype
    if act not in (torch.float32, torch.bfloat16):
        raise TypeError(f"activations must be float32 or bfloat16, got {act}")
    for name, t in (("k", k), ("v", v), ("a", a), ("b", b), ("out", out)):
        if t is not None and t.dtype != act:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {act} like q")
    if out is not None and (tuple(out.shape) != (N, Hv, V) or not out.is_contiguous()):
        raise ValueError(f"out must be a contiguous [{N}, {Hv}, {V}] tensor")
    if a is not None:
        _ab_strides(a, b, N, Hv, q.shape[1])
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (Hv,)
                              or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 [{Hv}] tensor")
    tile = (K, V) if _LAYOUTS[state_layout] == GDN_LAYOUT_KV else (V, K)
    if (state_pool.dtype not in (torch.float32, torch.bfloat16) or state_pool.dim() != 4
            or tuple(state_pool.shape[1:]) != (Hv,) + tile or not state_pool.is_contiguous()):
        raise ValueError(f"state_pool must be a contiguous float32 or bfloat16 [slots, {Hv}, "
                         f"{tile[0]}, {tile[1]}] tensor")
    if state_idx.dtype != torch.int32 or state_idx.dim() != 1 or not state_idx.is_contiguous():
        raise ValueError("state_idx must be a contiguous int32 [B] tensor")
    B = state_idx.shape[0]
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32
                                   or tuple(cu_seqlens.shape) != (B + 1,)
                                   or not cu_seqlens.is_contiguous()):
        raise ValueError("cu_seqlens must be a contiguous int32 [B+1] tensor")
    if intermediate_states is not None and (
            intermediate_states.dtype != state_pool.dtype
            or tuple(intermediate_states.shape) != (N, Hv) + tile
            or not intermediate_states.is_contiguous()):
        raise ValueError("intermediate_states must be a contiguous tensor of the pool's dtype "
                         "shaped like [N] + one pool row")
    dev = q.device
    for t in (k, v, a, b, A_log, dt_bias, state_pool, state_idx, cu_seqlens, out,
              intermediate_states):
        if t is not None and t.device != dev:
            raise ValueError("all tensors must be on the same device")
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU (ROCm device)")


def make_config(q, v, state_pool, state_idx, cu_seqlens=None, *, tokens_per_seq=None,
                scale: float = 0.0, eps: float = 1e-6, flags: int = 0, kernel_family: int = 0,
                block_v: int = 0, block_k: int = 0, waves_per_group: int = 0,
                k=None, state_layout=GDN_LAYOUT_KV, a=None, b=None) -> GdnConfig:
    """Sizes and strides of a call, read off the tensors' shapes."""
    import torch
    N, Hk, K = q.shape
    Hv, V = v.shape[1], v.shape[2]
    B = state_idx.shape[0]
    if tokens_per_seq is None:
        tokens_per_seq = N // B if (cu_seqlens is None and B > 0) else 1
    cfg = gdn_default_config()
    cfg.num_seqs = B
    cfg.tokens_per_seq = tokens_per_seq
    cfg.num_tokens = N
    cfg.num_k_heads, cfg.num_v_heads, cfg.head_k_dim, cfg.head_v_dim = Hk, Hv, K, V
    cfg.num_slots = state_pool.shape[0]
    cfg.state_layout = _LAYOUTS[state_layout]
    cfg.state_dtype = GDN_DTYPE_BF16 if state_pool.dtype == torch.bfloat16 else GDN_DTYPE_F32
    if q.dtype == torch.bfloat16:
        cfg.act_dtype = GDN_DTYPE_BF16
    elif q.dtype == torch.float32:
        cfg.act_dtype = GDN_DTYPE_F32
    else:
        cfg.act_dtype = -1  # rejected by the library with GDN_ERR_UNSUPPORTED_DTYPE
    cfg.scale = scale
    cfg.l2norm_eps = eps
    for name, t in (("q_stride_tok", q), ("k_stride_tok", q if k is None else k), ("v_stride_tok", v)):
        # strides of empty tensors and of size-1 dimensions are never used
        if t.shape[0] > 0 and (t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != t.shape[2])):
            raise ValueError("heads must be dense within a token (strides [*, D, 1])")
        setattr(cfg, name, t.stride(0) if t.shape[0] > 1 else 0)
    if a is not None:
        cfg.ab_stride_tok, cfg.ab_stride_khead = _ab_strides(a, b, N, Hv, Hk)
    cfg.flags = flags
    cfg.kernel_family = kernel_family
    cfg.block_v = block_v
    cfg.block_k = block_k
    cfg.waves_per_group = waves_per_group
    return cfg


def gdn_gating_delta_rule_update(q, k, v, a, b, A_log, dt_bias, state_pool, state_idx,
                                 cu_seqlens=None, out=None, intermediate_states=None, *,
                                 tokens_per_seq=None, scale: float = 0.0, eps: float = 1e-6,
                                 flags: int = 0, kernel_family: int = 0, block_v: int = 0,
                                 block_k: int = 0, waves_per_group: int = 0, stream=None,
                                 state_layout=GDN_LAYOUT_KV):
    """Enqueue the fused update on ``stream`` (default: torch's current stream
    on q's device).  Shapes: q, k [N, H_k, K]; v [N, H_v, V]; a, b [N, H_v];
    A_log, dt_bias [H_v] fp32; state_pool [slots, H_v, K, V] fp32 (updated in
    place); state_idx [B] int32; cu_seqlens [B+1] int32 or None; out [N, H_v, V]
    (allocated like v when None); intermediate_states [N, H_v, K, V] fp32 or
    None.  With state_layout "VK" (GDN_LAYOUT_VK) the pool is [slots, H_v, V, K]
    and intermediate_states [N, H_v, V, K].  Returns ``out``."""
    import torch
    if out is None:
        out = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    _check_tensors(q, k, v, a, b, A_log, dt_bias, state_pool, state_idx, cu_seqlens, out,
                   intermediate_states, state_layout)
    cfg = make_config(q, v, state_pool, state_idx, cu_seqlens, tokens_per_seq=tokens_per_seq,
                      scale=scale, eps=eps, flags=flags, kernel_family=kernel_family,
                      block_v=block_v, block_k=block_k, waves_per_group=waves_per_group, k=k,
                      state_layout=state_layout, a=a, b=b)
    stream = _stream_handle(stream, q.device)
    _check(raw_library().gdn_gating_delta_rule_update(
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
        _ptr(state_pool), _ptr(state_idx), _ptr(cu_seqlens), _ptr(out),
        _ptr(intermediate_states), ctypes.byref(cfg), stream))
    return out


class PreparedUpdate:
    """gdn_gating_delta_rule_update with its tensors bound once.  The checks,
    the config and the pointers are computed here, so each call only
    enqueues the launch: about 4 us of host time against 14 us for the
    function (measured at B = 1 on MI355X).  Meant for loops that reuse the
    same buffers: the contents of every tensor (state_idx and cu_seqlens
    included) may change between calls, their storage, shapes and strides
    may not.  The object holds references to the tensors."""

    def __init__(self, q, k, v, a, b, A_log, dt_bias, state_pool, state_idx, cu_seqlens=None,
                 out=None, intermediate_states=None, *, tokens_per_seq=None, scale: float = 0.0,
                 eps: float = 1e-6, flags: int = 0, kernel_family: int = 0, block_v: int = 0,
                 block_k: int = 0, waves_per_group: int = 0, state_layout=GDN_LAYOUT_KV):
        import torch
        if out is None:
            out = torch.empty(v.shape, dtype=v.dtype, device=v.device)
        _check_tensors(q, k, v, a, b, A_log, dt_bias, state_pool, state_idx, cu_seqlens, out,
                       intermediate_states, state_layout)
        self.cfg = make_config(q, v, state_pool, state_idx, cu_seqlens,
                               tokens_per_seq=tokens_per_seq, scale=scale, eps=eps, flags=flags,
                               kernel_family=kernel_family, block_v=block_v, block_k=block_k,
                               waves_per_group=waves_per_group, k=k, state_layout=state_layout,
                               a=a, b=b)
        self.out = out
        self._tensors = (q, k, v, a, b, A_log, dt_bias, state_pool, state_idx, cu_seqlens, out,
                         intermediate_states)
        self._device = q.device
        ptrs = [None if t is None else ctypes.c_void_p(t.data_ptr()) for t in self._tensors]
        lib = raw_library()
        _check(lib.gdn_validate(*ptrs, ctypes.byref(self.cfg)))
        self._fn = lib.gdn_gating_delta_rule_update
        self._args = (*ptrs, ctypes.byref(self.cfg))

    def __call__(self, stream=None):
        """Enqueue the update on ``stream`` (default: torch's current stream);
        returns ``out``."""
        _check(self._fn(*self._args, _stream_handle(stream, self._device)))
        return self.out


def gdn_chunk_gated_delta_rule_fwd(q, k, v, a, b, A_log, dt_bias, state_pool, state_idx,
                                   cu_seqlens=None, out=None, *, workspace=None,
                                   tokens_per_seq=None, scale: float = 0.0, eps: float = 1e-6,
                                   flags: int = 0, stream=None, state_layout=GDN_LAYOUT_KV):
    """The chunked forward (64-token chunks on the matrix cores): the outputs
    and final states of gdn_gating_delta_rule_update without intermediate
    states.  Arguments as there; K and V must be 32, 64 or 128.  workspace:
    None runs the one-kernel form; a CUDA tensor (any dtype, contiguous, at
    least gdn_chunk_workspace_bytes(...) bytes, see chunk_workspace) runs the
    two-kernel form over it.  Returns ``out``."""
    import torch
    if out is None:
        out = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    _check_tensors(q, k, v, a, b, A_log, dt_bias, state_pool, state_idx, cu_seqlens, out, None,
                   state_layout)
    cfg = make_config(q, v, state_pool, state_idx, cu_seqlens, tokens_per_seq=tokens_per_seq,
                      scale=scale, eps=eps, flags=flags, k=k, state_layout=state_layout, a=a, b=b)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q's device")
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    stream = _stream_handle(stream, q.device)
    _check(raw_library().gdn_chunk_gated_delta_rule_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
        _ptr(state_pool), _ptr(state_idx), _ptr(cu_seqlens), _ptr(out), ws_ptr, ws_bytes,
        ctypes.byref(cfg), stream))
    return out


def gdn_chunk_gated_delta_rule_fwd_noalloc(q, k, v, a, b, A_log, dt_bias, state_pool, state_idx,
                                           cu_seqlens, out, *, tokens_per_seq=None,
                                           scale: float = 0.0, eps: float = 1e-6, flags: int = 0,
                                           stream=None, state_layout=GDN_LAYOUT_KV):
    """The two-kernel chunked forward over the library's fixed device scratch
    (no workspace argument, nothing allocated by the call; ``out`` must be
    given).  Calls that may overlap on one GPU share that scratch and race.
    Returns ``out``."""
    _check_tensors(q, k, v, a, b, A_log, dt_bias, state_pool, state_idx, cu_seqlens, out, None,
                   state_layout)
    cfg = make_config(q, v, state_pool, state_idx, cu_seqlens, tokens_per_seq=tokens_per_seq,
                      scale=scale, eps=eps, flags=flags, k=k, state_layout=state_layout, a=a, b=b)
    stream = _stream_handle(stream, q.device)
    _check(raw_library().gdn_chunk_gated_delta_rule_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
        _ptr(state_pool), _ptr(state_idx), _ptr(cu_seqlens), _ptr(out), ctypes.byref(cfg), stream))
    return out


def gdn_chunk_workspace_bytes(cfg: GdnConfig) -> int:
    """Workspace bytes the two-kernel chunked form needs for cfg."""
    return int(raw_library().gdn_chunk_workspace_bytes(ctypes.byref(cfg)))


def chunk_workspace(q, v, state_pool, state_idx, cu_seqlens=None, *, tokens_per_seq=None):
    """A device byte tensor big enough to be the workspace of
    gdn_chunk_gated_delta_rule_fwd on these tensors (PyTorch allocates it)."""
    import torch
    cfg = make_config(q, v, state_pool, state_idx, cu_seqlens, tokens_per_seq=tokens_per_seq)
    return torch.empty(max(1, gdn_chunk_workspace_bytes(cfg)), dtype=torch.uint8, device=q.device)


def gdn_gating(a, b, A_log, dt_bias, g=None, beta=None, *, num_k_heads=None, stream=None):
    """The standalone gating step: g = -exp(A_log)*softplus(a + dt_bias) and
    beta = sigmoid(b), fp32 [N, H_v].  a, b: [N, H_v], or [N, H_k, G] views
    (then num_k_heads is taken from them).  Returns (g, beta)."""
    import torch
    if a.dim() == 3:
        N, Hk, G = a.shape
        Hv = Hk * G
    else:
        N, Hv = a.shape
        Hk = num_k_heads or Hv
    if g is None:
        g = torch.empty(N, Hv, dtype=torch.float32, device=a.device)
    if beta is None:
        beta = torch.empty(N, Hv, dtype=torch.float32, device=a.device)
    for name, t in (("g", g), ("beta", beta)):
        if t.dtype != torch.float32 or tuple(t.shape) != (N, Hv) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 [{N}, {Hv}] tensor")
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias)):
        if t.dtype != torch.float32 or tuple(t.shape) != (Hv,) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 [{Hv}] tensor")
    if a.device.type != "cuda" or any(t.device != a.device for t in (b, A_log, dt_bias, g, beta)):
        raise ValueError("tensors must live on one GPU")
    cfg = gdn_default_config()
    cfg.num_tokens = N
    cfg.num_k_heads, cfg.num_v_heads = Hk, Hv
    if a.dtype == torch.bfloat16:
        cfg.act_dtype = GDN_DTYPE_BF16
    elif a.dtype == torch.float32:
        cfg.act_dtype = GDN_DTYPE_F32
    else:
        raise TypeError(f"a/b must be float32 or bfloat16, got {a.dtype}")
    cfg.ab_stride_tok, cfg.ab_stride_khead = _ab_strides(a, b, N, Hv, Hk)
    stream = _stream_handle(stream, a.device)
    _check(raw_library().gdn_gating(_ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(g),
                                    _ptr(beta), ctypes.byref(cfg), stream))
    return g, beta


def gdn_recurrent_update(q, k, v, g, beta, state_pool, state_idx, cu_seqlens=None, out=None,
                         intermediate_states=None, *, tokens_per_seq=None, scale: float = 0.0,
                         eps: float = 1e-6, flags: int = 0, kernel_family: int = 0,
                         block_v: int = 0, block_k: int = 0, waves_per_group: int = 0,
                         stream=None, state_layout=GDN_LAYOUT_KV):
    """The update with precomputed gates (g, beta: fp32 [N, H_v], e.g. from
    gdn_gating).  Other arguments as gdn_gating_delta_rule_update."""
    import torch
    if out is None:
        out = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    N, Hv = v.shape[0], v.shape[1]
    for name, t in (("g", g), ("beta", beta)):
        if t.dtype != torch.float32 or tuple(t.shape) != (N, Hv) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 [{N}, {Hv}] tensor")
        if t.device != q.device:
            raise ValueError("all tensors must be on the same device")
    _check_tensors(q, k, v, None, None, None, None, state_pool, state_idx, cu_seqlens, out,
                   intermediate_states, state_layout)
    cfg = make_config(q, v, state_pool, state_idx, cu_seqlens, tokens_per_seq=tokens_per_seq,
                      scale=scale, eps=eps, flags=flags, kernel_family=kernel_family,
                      block_v=block_v, block_k=block_k, waves_per_group=waves_per_group, k=k,
                      state_layout=state_layout)
    stream = _stream_handle(stream, q.device)
    _check(raw_library().gdn_recurrent_update(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool), _ptr(state_idx),
        _ptr(cu_seqlens), _ptr(out), _ptr(intermediate_states), ctypes.byref(cfg), stream))
    return out


def gdn_validate(q, k, v, a, b, A_log, dt_bias, state_pool, state_idx, cu_seqlens=None,
                 out=None, intermediate_states=None, cfg: Optional[GdnConfig] = None, **kw) -> int:
    """Host-only argument check; returns the gdn_status code."""
    if cfg is None:
        cfg = make_config(q, v, state_pool, state_idx, cu_seqlens, k=k, **kw)
    return raw_library().gdn_validate(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log),
                             _ptr(dt_bias), _ptr(state_pool), _ptr(state_idx), _ptr(cu_seqlens),
                             _ptr(out), _ptr(intermediate_states), ctypes.byref(cfg))


def gdn_plan(cfg: GdnConfig, has_cu_seqlens: bool, has_intermediates: bool = False) -> GdnLaunchInfo:
    info = GdnLaunchInfo()
    _check(raw_library().gdn_plan(ctypes.byref(cfg), int(bool(has_cu_seqlens)),
                                  int(bool(has_intermediates)), ctypes.byref(info)))
    return info

