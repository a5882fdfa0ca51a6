"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and its host-side validation and planning behave as documented.
No call here launches a kernel or touches device memory (validation and
planning never dereference the pointers they are given)."""
import ctypes
import os
import re
import subprocess

import pytest

import linear_attention_recurrent_gating_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

# Fake, never-dereferenced device addresses (16-byte aligned).
A = [0x7f0000000000 + 0x100000 * i for i in range(12)]


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_exports_every_header_symbol():
    names = header_functions()
    assert set(names) == set(gdn.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (gdn_\w+)", out))
    missing = set(names) - exported
    assert not missing, f"declared in gdn.h but not exported: {missing}"
    lib = ctypes.CDLL(gdn.LIB_PATH)
    for n in names:
        assert hasattr(lib, n)


def test_header_and_c_example_compile_as_c11():
    """include/gdn.h is a C header: the plain-C example that drives the ABI
    compiles as C11 with every warning an error."""
    from linear_attention_recurrent_gating_amd import build
    r = subprocess.run(build.c_example_command(syntax_only=True), capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_abi_version_and_status_strings():
    assert gdn.gdn_abi_version() == 2
    seen = set()
    for code in range(0, 8):
        s = gdn.gdn_status_string(code)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 8
    assert gdn.gdn_status_string(99) == "unknown status"


def base_cfg(**kw):
    c = gdn.gdn_default_config()
    c.num_seqs, c.tokens_per_seq, c.num_tokens = 4, 1, 4
    c.num_k_heads, c.num_v_heads, c.head_k_dim, c.head_v_dim = 2, 4, 128, 128
    c.num_slots = 8
    c.act_dtype = gdn.GDN_DTYPE_BF16
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def validate(cfg, ptrs=None, cu=None, inter=None):
    p = list(A[:11]) if ptrs is None else ptrs
    lib = gdn.raw_library()
    return lib.gdn_validate(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], cu, p[10],
                            inter, ctypes.byref(cfg))


def test_defaults():
    c = gdn.gdn_default_config()
    assert c.tokens_per_seq == 1 and c.scale == 0.0 and abs(c.l2norm_eps - 1e-6) < 1e-12
    assert c.q_stride_tok == 0 and c.block_v == 0 and c.waves_per_group == 0 and c.flags == 0


def test_valid_config_passes():
    assert validate(base_cfg()) == gdn.GDN_OK
    assert gdn.gdn_last_error_message() == ""


@pytest.mark.parametrize("field,value,code", [
    ("num_seqs", -1, 2),
    ("num_k_heads", 0, 2),
    ("num_v_heads", 3, 2),          # not a multiple of H_k = 2
    ("head_k_dim", 96, 3),
    ("head_v_dim", 48, 3),
    ("head_k_dim", 512, 3),
    ("act_dtype", 2, 4),
    ("tokens_per_seq", 0, 2),
    ("num_tokens", 3, 2),           # < B*T
    ("num_slots", 0, 2),
    ("l2norm_eps", -1.0, 7),
    ("scale", float("nan"), 7),
    ("q_stride_tok", 100, 2),       # below dense 2*128
    ("k_stride_tok", 260, 5),       # not a multiple of 8
    ("v_stride_tok", 516, 5),
    ("block_v", 12, 7),
    ("block_v", 256, 7),
    ("waves_per_group", 9, 7),
    ("waves_per_group", 3, 7),      # row split: not a multiple of the 4 waves per head
    ("kernel_family", 3, 7),        # value rows need the VK layout
    ("kernel_family", 5, 7),
    ("state_layout", 2, 7),
    ("block_k", 48, 7),             # no row-split kernel with 48 rows per wave
])
def test_invalid_config(field, value, code):
    c = base_cfg(**{field: value})
    assert validate(c) == code
    assert gdn.gdn_last_error_message() != ""


def test_unsupported_block_for_k():
    # K = 256 with 64-column tiles would need 256 state VGPRs per lane
    assert validate(base_cfg(head_k_dim=256, block_v=64)) == 7
    # column tiles: waves must divide G*V/block_v = 8
    assert validate(base_cfg(kernel_family=gdn.GDN_KERNEL_COLUMN_TILES, waves_per_group=3)) == 7
    # the row-split kernel takes any number of tokens per sequence
    assert validate(base_cfg(kernel_family=gdn.GDN_KERNEL_ROW_SPLIT, tokens_per_seq=2,
                             num_tokens=8)) == 0
    assert validate(base_cfg(kernel_family=gdn.GDN_KERNEL_ROW_SPLIT, block_v=32)) == 7
    # column tiles cover all K rows
    assert validate(base_cfg(kernel_family=gdn.GDN_KERNEL_COLUMN_TILES, block_k=32)) == 7


def test_null_pointers():
    for i in [0, 1, 2, 3, 4, 5, 6, 7, 8, 10]:
        p = list(A[:11])
        p[i] = None
        assert validate(base_cfg(), ptrs=p) == 1, f"pointer {i}"


def test_empty_batch_accepts_null_pointers():
    c = base_cfg(num_seqs=0, num_tokens=0)
    assert validate(c, ptrs=[None] * 11) == gdn.GDN_OK
    # sequences that are all zero-length (cu_seqlens all 0): nothing is read
    c = base_cfg(num_seqs=3, num_tokens=0)
    assert validate(c, ptrs=[None] * 11, cu=A[11]) == gdn.GDN_OK


def test_misaligned_pointers():
    for i in [0, 1, 2, 7, 10]:
        p = list(A[:11])
        p[i] += 8
        assert validate(base_cfg(), ptrs=p) == 5, f"pointer {i}"
    p = list(A[:11])
    p[3] += 1  # a: bf16 needs 2-byte alignment
    assert validate(base_cfg(), ptrs=p) == 5
    p = list(A[:11])
    p[3] += 2  # fine for bf16
    assert validate(base_cfg(), ptrs=p) == 0
    assert validate(base_cfg(act_dtype=gdn.GDN_DTYPE_F32), ptrs=p) == 5
    assert validate(base_cfg(), inter=A[11] + 4) == 5


def test_varlen_ignores_tokens_per_seq():
    c = base_cfg(tokens_per_seq=0, num_tokens=37)
    assert validate(c, cu=A[9]) == 0
    assert validate(c) == 2


def test_plan_tile_table():
    decode = gdn.gdn_plan(base_cfg(num_seqs=512, num_tokens=512, num_k_heads=16, num_v_heads=32,
                                   num_slots=4096), False)
    assert decode.multi_token == 0 and decode.tokens_per_chunk == 1
    assert decode.kernel_family == gdn.GDN_KERNEL_ROW_SPLIT
    assert decode.block_v == 128                   # whole rows per wavefront
    assert decode.block_k == 64                    # 32 rows per lane: 2 waves per head
    assert decode.waves_per_group == 4 and decode.threads_per_group == 256
    assert decode.workgroups == 512 * 16          # one per (sequence, k-head)
    assert decode.lds_bytes == (2 * 128 + 4 * (2 * 128 + 4)) * 4
    # a smaller batch: the same tile (32 rows per lane, the k-head's two heads)
    small = gdn.gdn_plan(base_cfg(num_seqs=64, num_tokens=64, num_k_heads=16, num_v_heads=32,
                                  num_slots=1024), False)
    assert small.block_k == 64 and small.waves_per_group == 4 and small.workgroups == 64 * 16
    # K = V = 256, one token: 32 rows per lane, 8 wavefronts per head (one
    # 256-float row per instruction)
    big = gdn.gdn_plan(base_cfg(head_k_dim=256, head_v_dim=256), False)
    assert big.kernel_family == gdn.GDN_KERNEL_ROW_SPLIT and big.block_k == 32
    assert big.waves_per_group == 8 and big.workgroups == 4 * 2 * 2
    # other shapes, one token: 32 rows per lane with fp32 state, 16 with bf16
    k64 = gdn.gdn_plan(base_cfg(head_k_dim=64), False)       # V = 128: 2 rows per instruction
    assert k64.kernel_family == gdn.GDN_KERNEL_ROW_SPLIT and k64.block_k == 64
    k64b = gdn.gdn_plan(base_cfg(head_k_dim=64, state_dtype=gdn.GDN_DTYPE_BF16), False)
    assert k64b.block_k == 64        # a small grid: 32 rows per lane with bf16 state too
    k64w = gdn.gdn_plan(base_cfg(head_k_dim=64, state_dtype=gdn.GDN_DTYPE_BF16, num_seqs=1024,
                                 num_tokens=1024, num_slots=1024), False)
    assert k64w.block_k == 32        # 2048 workgroups: 16 rows per lane
    spec = gdn.gdn_plan(base_cfg(num_seqs=128, num_tokens=512, num_k_heads=16, num_v_heads=32,
                                 num_slots=1024), True)
    assert spec.multi_token == 1 and spec.tokens_per_chunk >= 2
    assert spec.kernel_family == gdn.GDN_KERNEL_ROW_SPLIT and spec.block_k == 64
    assert spec.waves_per_group == 4             # 2 heads x 2 wavefronts of 64 rows
    spec16 = gdn.gdn_plan(base_cfg(num_seqs=128, num_tokens=512, num_k_heads=16, num_v_heads=32,
                                   num_slots=1024, state_dtype=gdn.GDN_DTYPE_BF16), True)
    assert spec16.kernel_family == gdn.GDN_KERNEL_ROW_SPLIT and spec16.block_k == 64
    for sd in (gdn.GDN_DTYPE_F32, gdn.GDN_DTYPE_BF16):   # column tiles: 64 columns either way
        cols = gdn.gdn_plan(base_cfg(num_seqs=128, num_tokens=512, num_k_heads=16, num_v_heads=32,
                                     num_slots=1024, state_dtype=sd,
                                     kernel_family=gdn.GDN_KERNEL_COLUMN_TILES), True)
        assert cols.block_v == 64 and cols.waves_per_group == 4   # G * V / 64 tile units
    multi = gdn.gdn_plan(base_cfg(tokens_per_seq=4, num_tokens=16), False)
    assert multi.multi_token == 1
    # bf16 state: the same 32 rows per lane from 256 (sequence, k-head) pairs on
    dec16 = gdn.gdn_plan(base_cfg(state_dtype=gdn.GDN_DTYPE_BF16, num_seqs=16, num_tokens=16,
                                  num_k_heads=16, num_v_heads=32, num_slots=16), False)
    assert dec16.kernel_family == gdn.GDN_KERNEL_ROW_SPLIT and dec16.block_k == 64   # 32 rows per lane
    # fewer pairs: 8 rows per lane, one head per 8-wavefront workgroup
    tiny = gdn.gdn_plan(base_cfg(state_dtype=gdn.GDN_DTYPE_BF16), False)
    assert tiny.block_k == 16 and tiny.waves_per_group == 8 and tiny.workgroups == 4 * 2 * 2
    # G = 3 (H_k = 2, H_v = 6) with V = 32, BV = 32: 3 wave units per k-head
    odd = gdn.gdn_plan(base_cfg(num_v_heads=6, head_v_dim=32,
                                kernel_family=gdn.GDN_KERNEL_COLUMN_TILES), True)
    assert odd.waves_per_group == 3 and odd.workgroups == 4 * 2
    # row split with G = 3, K = V = 128, a small grid: 8 waves per head, one head per group
    odd_rows = gdn.gdn_plan(base_cfg(num_v_heads=6), False)
    assert odd_rows.kernel_family == gdn.GDN_KERNEL_ROW_SPLIT and odd_rows.block_k == 16
    assert odd_rows.waves_per_group == 8 and odd_rows.workgroups == 4 * 2 * 3
    # a larger grid: 2 waves per head, all three heads in a group
    odd_big = gdn.gdn_plan(base_cfg(num_v_heads=6, num_seqs=128, num_tokens=128, num_slots=128),
                           False)
    assert odd_big.block_k == 64 and odd_big.waves_per_group == 6 and odd_big.workgroups == 128 * 2
    # 16 rows per lane when asked for four waves per workgroup
    odd4 = gdn.gdn_plan(base_cfg(num_v_heads=6, waves_per_group=4), False)
    assert odd4.block_k == 32 and odd4.workgroups == 4 * 2 * 3
    forced = gdn.gdn_plan(base_cfg(block_v=16, waves_per_group=4), False)
    assert forced.kernel_family == gdn.GDN_KERNEL_COLUMN_TILES
    assert forced.block_v == 16 and forced.waves_per_group == 4 and forced.block_k == 128
    assert forced.workgroups == 4 * 2 * (2 * 8 // 4)
    # row split, 16 rows per wavefront (8 rows per lane): 8 waves per head
    r16 = gdn.gdn_plan(base_cfg(block_k=16), False)
    assert r16.kernel_family == gdn.GDN_KERNEL_ROW_SPLIT and r16.block_k == 16
    assert r16.waves_per_group == 8 and r16.workgroups == 4 * 2 * 2
    # row split, one head per workgroup
    r1 = gdn.gdn_plan(base_cfg(waves_per_group=2), False)
    assert r1.kernel_family == gdn.GDN_KERNEL_ROW_SPLIT and r1.block_k == 64
    assert r1.waves_per_group == 2 and r1.workgroups == 4 * 2 * 2
    # forcing column tiles for a single token
    c1 = gdn.gdn_plan(base_cfg(kernel_family=gdn.GDN_KERNEL_COLUMN_TILES), False)
    assert c1.kernel_family == gdn.GDN_KERNEL_COLUMN_TILES and c1.block_v == 64


def test_plan_row_split_token_loop():
    """The row split over several tokens: 16 staged tokens of q/k (shared),
    of v (per head) and double-buffered partial sums in LDS."""
    R = gdn.GDN_KERNEL_ROW_SPLIT
    pl = gdn.gdn_plan(base_cfg(kernel_family=R, tokens_per_seq=4, num_tokens=16), True)
    assert pl.kernel_family == R and pl.multi_token == 1 and pl.tokens_per_chunk == 16
    assert pl.block_k == 16 and pl.waves_per_group == 8 and pl.workgroups == 4 * 2 * 2
    assert pl.lds_bytes == (2 * 16 * 128 + 1 * 16 * 128 + 2 * 8 * (2 * 128 + 4)) * 4
    two = gdn.gdn_plan(base_cfg(kernel_family=R, tokens_per_seq=4, num_tokens=16, block_k=64), True)
    assert two.waves_per_group == 4 and two.workgroups == 4 * 2     # two heads per workgroup
    assert two.lds_bytes == (2 * 16 * 128 + 2 * 16 * 128 + 2 * 4 * (2 * 128 + 4)) * 4
    # K = V = 256 would need more than 64 KiB of LDS
    big = base_cfg(kernel_family=R, tokens_per_seq=4, num_tokens=16, head_k_dim=256, head_v_dim=256)
    assert validate(big) == 7
    # rows per lane of the token loop: 32 from 512 (sequence, k-head) workgroups,
    # or from 256 when intermediate states are written (with bf16 state: for
    # >= 8 tokens per sequence); 8 below
    heads = dict(num_k_heads=16, num_v_heads=32)
    def bk(B, T, inter, **kw):
        cfg = base_cfg(num_seqs=B, tokens_per_seq=T, num_tokens=B * T, num_slots=B, **heads, **kw)
        return gdn.gdn_plan(cfg, False, inter).block_k
    bf16 = dict(state_dtype=gdn.GDN_DTYPE_BF16)
    assert bk(32, 4, False) == 64 and bk(32, 4, True) == 64
    assert bk(16, 4, False) == 16 and bk(16, 4, True) == 64
    assert bk(16, 4, True, **bf16) == 16 and bk(16, 7, True, **bf16) == 16
    assert bk(16, 8, True, **bf16) == 64 and bk(16, 16, True) == 64
    assert bk(8, 16, True) == 16
    # other head dims
    def plan(B, T, inter, K, V, **kw):
        cfg = base_cfg(num_seqs=B, tokens_per_seq=T, num_tokens=B * T, num_slots=B, head_k_dim=K,
                       head_v_dim=V, **heads, **kw)
        return gdn.gdn_plan(cfg, False, inter)
    assert plan(16, 4, False, 256, 128).block_k == 64        # K = 256, V = 128: 32 rows per lane
    assert plan(16, 4, True, 64, 128).block_k == 32          # fp32 intermediates: 16 rows per lane
    assert plan(16, 4, True, 64, 128, state_dtype=gdn.GDN_DTYPE_BF16).block_k == 16
    # no intermediates, >= 1024 (sequence, k-head) workgroups: the column tiles
    assert plan(64, 4, False, 128, 64).kernel_family == gdn.GDN_KERNEL_COLUMN_TILES
    assert plan(32, 4, False, 128, 64).kernel_family == R
    assert plan(64, 4, True, 128, 64).kernel_family == R
    assert plan(64, 4, False, 128, 128).kernel_family == R
    cols = plan(64, 4, False, 128, 64)           # fp32 state at K = 128, V = 64: 32 columns
    assert cols.block_v == 32 and cols.waves_per_group == 4
    assert plan(64, 4, False, 128, 64, state_dtype=gdn.GDN_DTYPE_BF16).block_v == 64


def test_plan_value_rows():
    vk = gdn.gdn_plan(base_cfg(state_layout=gdn.GDN_LAYOUT_VK, num_seqs=512, num_tokens=512,
                               num_k_heads=16, num_v_heads=32), False)
    assert vk.kernel_family == gdn.GDN_KERNEL_VALUE_ROWS
    assert vk.block_v == 32 and vk.block_k == 128      # 32 whole value-rows per wavefront
    assert vk.waves_per_group == 8 and vk.workgroups == 512 * 16 and vk.lds_bytes == 0
    vk16 = gdn.gdn_plan(base_cfg(state_layout=gdn.GDN_LAYOUT_VK, num_seqs=512, num_tokens=512,
                                 num_k_heads=16, num_v_heads=32,
                                 state_dtype=gdn.GDN_DTYPE_BF16), False)
    assert vk16.waves_per_group == 4 and vk16.workgroups == 512 * 16 * 2   # bf16: 4 waves
    multi = gdn.gdn_plan(base_cfg(state_layout=gdn.GDN_LAYOUT_VK, tokens_per_seq=4,
                                  num_tokens=16), True)
    assert multi.kernel_family == gdn.GDN_KERNEL_VALUE_ROWS and multi.multi_token == 1
    w4 = gdn.gdn_plan(base_cfg(state_layout=gdn.GDN_LAYOUT_VK, waves_per_group=4), False)
    assert w4.waves_per_group == 4 and w4.workgroups == 4 * 2 * 2
    assert validate(base_cfg(state_layout=gdn.GDN_LAYOUT_VK, block_v=32)) == 7
    assert validate(base_cfg(state_layout=gdn.GDN_LAYOUT_VK,
                             kernel_family=gdn.GDN_KERNEL_ROW_SPLIT)) == 7
    assert validate(base_cfg(state_layout=gdn.GDN_LAYOUT_VK, waves_per_group=3)) == 7
    # K = V = 256: 16 wavefronts per head, spread over two 8-wave workgroups
    big = gdn.gdn_plan(base_cfg(state_layout=gdn.GDN_LAYOUT_VK, head_k_dim=256,
                                head_v_dim=256), False)
    assert big.block_v == 16 and big.waves_per_group == 8 and big.workgroups == 4 * 2 * 4


def test_plan_chunked():
    ck = gdn.gdn_plan(base_cfg(kernel_family=gdn.GDN_KERNEL_CHUNKED, tokens_per_seq=100,
                               num_tokens=400), False)
    assert ck.kernel_family == gdn.GDN_KERNEL_CHUNKED and ck.multi_token == 1
    assert ck.tokens_per_chunk == 64 and ck.block_v == 16 and ck.block_k == 128
    assert ck.waves_per_group == 8 and ck.workgroups == 4 * 4 and ck.threads_per_group == 512
    assert 64 * 1024 < ck.lds_bytes <= 160 * 1024
    # either layout and state dtype; V = 64 takes four wavefronts of 16 columns
    vk = gdn.gdn_plan(base_cfg(kernel_family=gdn.GDN_KERNEL_CHUNKED, head_v_dim=64,
                               state_layout=gdn.GDN_LAYOUT_VK, state_dtype=gdn.GDN_DTYPE_BF16),
                      True)
    assert vk.kernel_family == gdn.GDN_KERNEL_CHUNKED and vk.waves_per_group == 4
    f32 = gdn.gdn_plan(base_cfg(kernel_family=gdn.GDN_KERNEL_CHUNKED,
                                act_dtype=gdn.GDN_DTYPE_F32), False)
    assert f32.lds_bytes <= 160 * 1024
    chunked = dict(kernel_family=gdn.GDN_KERNEL_CHUNKED)
    assert validate(base_cfg(head_k_dim=256, **chunked)) == 3
    assert validate(base_cfg(head_v_dim=256, **chunked)) == 3
    for over in ("block_v", "block_k", "waves_per_group"):
        assert validate(base_cfg(**{over: 32 if over != "waves_per_group" else 4}, **chunked)) == 7
    # no per-token states
    assert validate(base_cfg(**chunked), inter=A[11]) == 7
    assert validate(base_cfg(**chunked)) == 0
    # 64 rows of a 2^25-element token stride (bf16) span 4 GiB: offsets would overflow
    assert validate(base_cfg(k_stride_tok=1 << 25, **chunked)) == 3
    # AUTO takes the chunked kernel from 32 tokens per sequence on average,
    # unless intermediate states are written or a tiling override is given
    long = base_cfg(tokens_per_seq=4096, num_tokens=4 * 4096)
    assert gdn.gdn_plan(long, False).kernel_family == gdn.GDN_KERNEL_CHUNKED
    # with intermediate states on 8 (sequence, k-head) pairs: 16-column tiles
    tiny_inter = gdn.gdn_plan(long, False, True)
    assert tiny_inter.kernel_family == gdn.GDN_KERNEL_COLUMN_TILES and tiny_inter.block_v == 16
    assert tiny_inter.waves_per_group == 2
    wide_inter = gdn.gdn_plan(base_cfg(tokens_per_seq=64, num_tokens=64 * 64, num_seqs=64,
                                       num_slots=64, num_k_heads=16, num_v_heads=32), False, True)
    assert wide_inter.kernel_family == gdn.GDN_KERNEL_ROW_SPLIT
    assert gdn.gdn_plan(base_cfg(tokens_per_seq=4096, num_tokens=4 * 4096, block_v=32),
                        False).kernel_family == gdn.GDN_KERNEL_COLUMN_TILES
    # more (sequence, v-head) workgroups than CUs: from 32 tokens on
    wide = dict(num_seqs=128, num_k_heads=16, num_v_heads=32, num_slots=256)
    at32 = base_cfg(tokens_per_seq=32, num_tokens=128 * 32, **wide)
    assert gdn.gdn_plan(at32, False).kernel_family == gdn.GDN_KERNEL_CHUNKED
    below = base_cfg(tokens_per_seq=31, num_tokens=128 * 31, **wide)
    assert gdn.gdn_plan(below, False).kernel_family == gdn.GDN_KERNEL_ROW_SPLIT
    # at most one workgroup per CU (256): from 16 tokens on
    one_wave = dict(num_seqs=8, num_k_heads=16, num_v_heads=32, num_slots=16)
    assert gdn.gdn_plan(base_cfg(tokens_per_seq=16, num_tokens=8 * 16, **one_wave),
                        False).kernel_family == gdn.GDN_KERNEL_CHUNKED
    assert gdn.gdn_plan(base_cfg(tokens_per_seq=15, num_tokens=8 * 15, **one_wave),
                        False).kernel_family == gdn.GDN_KERNEL_ROW_SPLIT
    nine = dict(one_wave, num_seqs=9)     # 288 workgroups: the 32-token rule again
    assert gdn.gdn_plan(base_cfg(tokens_per_seq=16, num_tokens=9 * 16, **nine),
                        False).kernel_family == gdn.GDN_KERNEL_ROW_SPLIT
    # smaller states cross over later: 32 * sqrt(128 * 128 / (K * V)) tokens
    for (K, V), need in (((128, 64), 46), ((64, 64), 64), ((32, 32), 128)):
        at = base_cfg(tokens_per_seq=need, num_tokens=128 * need, head_k_dim=K, head_v_dim=V, **wide)
        assert gdn.gdn_plan(at, False).kernel_family == gdn.GDN_KERNEL_CHUNKED, (K, V)
        less = base_cfg(tokens_per_seq=need - 1, num_tokens=128 * (need - 1), head_k_dim=K,
                        head_v_dim=V, **wide)
        assert gdn.gdn_plan(less, False).kernel_family != gdn.GDN_KERNEL_CHUNKED, (K, V)
    # varlen: the mean length decides (num_tokens / num_seqs)
    assert gdn.gdn_plan(base_cfg(num_tokens=4 * 40), True).kernel_family == gdn.GDN_KERNEL_CHUNKED
    # no chunked instance for K = 256: AUTO falls back without an error
    big = gdn.gdn_plan(base_cfg(head_k_dim=256, tokens_per_seq=100, num_tokens=400), False)
    assert big.kernel_family == gdn.GDN_KERNEL_ROW_SPLIT and gdn.gdn_last_error_message() == ""
    # nor a row-split token loop within the LDS budget at K = V = 256: column tiles
    huge = gdn.gdn_plan(base_cfg(head_k_dim=256, head_v_dim=256, tokens_per_seq=100,
                                 num_tokens=400), False)
    assert huge.kernel_family == gdn.GDN_KERNEL_COLUMN_TILES


def test_auto_counts_processed_tokens():
    """Without cu_seqlens only num_seqs * tokens_per_seq rows belong to
    sequences: a one-token decode over a larger token buffer stays on the
    single-token row split, and the chunked threshold counts the processed
    tokens, not the buffer's rows."""
    dec = gdn.gdn_plan(base_cfg(num_seqs=8, tokens_per_seq=1, num_tokens=512, num_slots=8), False)
    assert dec.kernel_family == gdn.GDN_KERNEL_ROW_SPLIT and dec.multi_token == 0
    few = gdn.gdn_plan(base_cfg(num_seqs=8, tokens_per_seq=4, num_tokens=4096, num_slots=8,
                                num_k_heads=16, num_v_heads=32), False)
    assert few.kernel_family == gdn.GDN_KERNEL_ROW_SPLIT and few.multi_token == 1


def test_chunked_ab_stride_offsets():
    """The chunked kernel addresses 64 token rows of a and b with 32-bit
    offsets: an a/b token stride whose 64 rows span 2 GiB or more is
    rejected for the chunked family, and AUTO falls back to a per-token
    kernel (64-bit row addressing) without an error."""
    chunked = dict(kernel_family=gdn.GDN_KERNEL_CHUNKED, tokens_per_seq=100, num_tokens=400)
    big = (1 << 26) + 5          # bf16: 64 rows of it span just over 8 GiB
    assert validate(base_cfg(ab_stride_tok=big, **chunked)) == 3
    assert "2 GiB" in gdn.gdn_last_error_message()
    assert validate(base_cfg(ab_stride_tok=(1 << 23) - 64, **chunked)) == 0   # just under 1 GiB
    auto = gdn.gdn_plan(base_cfg(ab_stride_tok=big, tokens_per_seq=100, num_tokens=400), False)
    assert auto.kernel_family != gdn.GDN_KERNEL_CHUNKED and gdn.gdn_last_error_message() == ""


def test_chunked_entry_point_validation():
    lib = gdn.raw_library()

    def call(c, out=A[10], ws=None, ws_bytes=0):
        return lib.gdn_chunk_gated_delta_rule_fwd(*A[:7], A[7], A[8], None, out, ws, ws_bytes,
                                                  None if c is None else ctypes.byref(c), None)
    assert call(base_cfg(kernel_family=gdn.GDN_KERNEL_ROW_SPLIT)) == 7
    assert call(base_cfg(head_k_dim=256)) == 3
    assert call(base_cfg(), out=None) == 1
    assert call(None) == 1
    # a zero-sequence batch returns before touching anything
    assert call(base_cfg(num_seqs=0, num_tokens=0)) == 0


def test_chunk_workspace_size_and_checks():
    """The workspace of the two-kernel form: one 21,760-byte entry per (chunk
    slot, v-head), floor(N / 64) + B slots; a workspace that is too small or
    not 256-byte aligned is rejected before any launch."""
    lib = gdn.raw_library()
    entry = 21760
    c = base_cfg(num_seqs=3, tokens_per_seq=100, num_tokens=300)   # 4 v-heads
    need = gdn.gdn_chunk_workspace_bytes(c)
    assert need == (300 // 64 + 3) * 4 * entry
    assert gdn.gdn_chunk_workspace_bytes(base_cfg(num_seqs=0, num_tokens=0)) == 0
    assert lib.gdn_chunk_workspace_bytes(None) == 0
    ws = 0x7f1000000000            # fake, never dereferenced; 256-byte aligned

    def call(ws_ptr, nbytes):
        return lib.gdn_chunk_gated_delta_rule_fwd(*A[:7], A[7], A[8], None, A[10], ws_ptr, nbytes,
                                                  ctypes.byref(c), None)
    assert call(ws, need - 1) == 7
    assert "needs" in gdn.gdn_last_error_message()
    assert call(ws + 128, need) == 5
    # a varlen call: every sequence may start a new slot
    v = base_cfg(num_seqs=5, num_tokens=129, num_slots=8)
    assert gdn.gdn_chunk_workspace_bytes(v) == (129 // 64 + 5) * 4 * entry


def test_ab_stride_validation():
    assert validate(base_cfg(ab_stride_khead=1)) == 2            # below G = 2
    assert validate(base_cfg(ab_stride_khead=4, ab_stride_tok=5)) == 2   # below (H_k-1)*4 + 2 = 6
    assert validate(base_cfg(ab_stride_khead=4, ab_stride_tok=8)) == 0
    lib = gdn.raw_library()
    c = base_cfg(ab_stride_khead=1)
    assert lib.gdn_gating(A[0], A[1], A[2], A[3], A[4], A[5], ctypes.byref(c), None) == 2
    c = base_cfg()
    assert lib.gdn_gating(A[0], None, A[2], A[3], A[4], A[5], ctypes.byref(c), None) == 1
    assert lib.gdn_gating(A[0], A[1], A[2], A[3], A[4] + 2, A[5], ctypes.byref(c), None) == 5
    assert lib.gdn_recurrent_update(A[0], A[1], A[2], None, A[4], A[5], A[6], None, A[7], None,
                                    ctypes.byref(c), None) == 1


def test_binding_rejects_bad_tensors_on_cpu():
    import torch
    q = torch.zeros(2, 1, 32)
    v = torch.zeros(2, 2, 32)
    ab = torch.zeros(2, 2)
    pars = torch.zeros(2)
    pool = torch.zeros(4, 2, 32, 32)
    idx = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        gdn.gdn_gating_delta_rule_update(q, q, v, ab, ab, pars, pars, pool, idx)
    with pytest.raises(ValueError, match="state_idx"):
        gdn.gdn_gating_delta_rule_update(q, q, v, ab, ab, pars, pars, pool, idx.long())
    with pytest.raises(TypeError):
        gdn.gdn_gating_delta_rule_update(q, q, v.double(), ab, ab, pars, pars, pool, idx)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(gdn, "LIB_PATH", str(tmp_path / "libgdn.so"))
    with pytest.raises(ImportError, match="not built"):
        gdn._load()


def test_noalloc_entry_point_rejections():
    """The allocation-free chunked entry point checks its arguments, and that
    the call fits the library's 128 MiB scratch, before it looks at any
    device: a call needing more is rejected with GDN_ERR_BAD_ARGUMENT."""
    lib = gdn.raw_library()

    def call(c, out=A[10]):
        return lib.gdn_chunk_gated_delta_rule_fwd_noalloc(*A[:7], A[7], A[8], None, out,
                                                          None if c is None else ctypes.byref(c),
                                                          None)
    assert call(None) == 1
    assert call(base_cfg(kernel_family=gdn.GDN_KERNEL_ROW_SPLIT)) == 7
    assert call(base_cfg(head_k_dim=256)) == 3
    assert call(base_cfg(), out=None) == 1
    assert call(base_cfg(num_seqs=0, num_tokens=0)) == 0
    big = base_cfg(num_seqs=2, tokens_per_seq=64 * 800, num_tokens=2 * 64 * 800, num_slots=4)
    assert gdn.gdn_chunk_workspace_bytes(big) > 128 << 20
    assert call(big) == 7
    assert "scratch" in gdn.gdn_last_error_message()
