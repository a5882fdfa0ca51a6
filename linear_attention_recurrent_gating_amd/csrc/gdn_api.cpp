// C-ABI of libgdn: argument validation, the tile table and the launch.
// The operation and its conventions are documented in include/gdn.h.

#include "gdn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "gdn_internal.h"

namespace {

thread_local char g_last_error[512] = "";

gdn_status fail(gdn_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

bool supported_dim(int d) { return d == 32 || d == 64 || d == 128 || d == 256; }

int default_block_v(const gdn_config& c) {
    // 64 columns (a 256-byte fp32 or 128-byte bf16 row segment, 128 state
    // VGPRs at K = 128), measured on MI355X against 32: spec verify 276 vs
    // 300 us with fp32 state, 202 vs 237 us with bf16. 32 for fp32 state at
    // K = 128, V = 64 (64 x 4 tokens 25.8 vs 30.6 us, 256 x 16 166.8 vs
    // 176.2 us). Narrower where V or the instance table asks for it.
    int bv = (c.state_dtype == GDN_DTYPE_F32 && c.head_k_dim == 128 && c.head_v_dim == 64) ? 32 : 64;
    while (bv > 8 && (c.head_v_dim % bv != 0 || !gdn::instance_exists(c.head_k_dim, bv))) bv /= 2;
    return bv;
}

// Dynamic LDS a per-token kernel may ask for (the default launch limit).
constexpr int kMaxDynamicLds = 64 * 1024;

// Largest divisor of `units` (wave units per k-head) not above `max_waves`.
int default_waves(int units, int max_waves = 8) {
    for (int w = max_waves; w >= 1; --w)
        if (units % w == 0) return w;
    return 1;
}

// The chunked kernel's launch for a config, or the reason it has none.
gdn_status chunked_shape(const gdn_config& c, gdn::LaunchShape& s) {
    const int K = c.head_k_dim, V = c.head_v_dim;
    if (c.block_v != 0 || c.block_k != 0 || c.waves_per_group != 0)
        return fail(GDN_ERR_BAD_ARGUMENT, "the chunked kernel takes no tiling overrides "
                                          "(block_v, block_k, waves_per_group must be 0)");
    const int bytes = gdn::chunk_lds_bytes(K, V, c.act_dtype);
    if (bytes == 0)
        return fail(GDN_ERR_UNSUPPORTED_SHAPE, "no chunked kernel for K = %d, V = %d "
                                               "(each must be 32, 64 or 128)", K, V);
    // Buffer offsets within one chunk are 32-bit.
    const int64_t esize = c.act_dtype == GDN_DTYPE_F32 ? 4 : 2;
    const int64_t rows[] = {c.q_stride_tok ? c.q_stride_tok : int64_t(c.num_k_heads) * K,
                            c.k_stride_tok ? c.k_stride_tok : int64_t(c.num_k_heads) * K,
                            c.v_stride_tok ? c.v_stride_tok : int64_t(c.num_v_heads) * V,
                            int64_t(c.num_v_heads) * V,
                            c.ab_stride_tok ? c.ab_stride_tok : int64_t(c.num_v_heads)};
    for (int64_t r : rows)
        if (r * esize * gdn::kChunkedTokens >= (int64_t(1) << 31))
            return fail(GDN_ERR_UNSUPPORTED_SHAPE, "64 token rows of %lld elements exceed 2 GiB",
                        static_cast<long long>(r));
    s.kind = gdn::kKindChunked;
    s.multi_token = 1;
    s.chunk = gdn::kChunkedTokens;
    s.block_v = gdn::chunk_block_v();
    s.block_k = K;
    s.rows_rpl_max = 0;
    s.waves = V / s.block_v;
    s.groups = static_cast<int64_t>(c.num_seqs) * c.num_v_heads;
    if (s.groups > INT32_MAX)
        return fail(GDN_ERR_BAD_SHAPE, "grid of %lld workgroups is too large",
                    static_cast<long long>(s.groups));
    s.lds_bytes = bytes;
    return GDN_OK;
}

// GDN_KERNEL_AUTO takes the chunked kernel for calls that write no
// intermediate states, when it has an instance for the shape, and the
// sequences average at least
//   * 32 tokens: its 64-token chunks beat the per-token loop from there on
//     (MI355X, H 16/32, K = V = 128: 64 x 32 tokens 120 vs 164 us, 256 x 32
//     443 vs 567 us; 64 x 16 118 vs 98 us the other way), or
//   * 16 tokens when the (sequence, v-head) workgroups fit one per CU: the
//     chunks then run as one wave (8 x 16 tokens 18.6 vs 23.2 us; 16 x 16
//     34.4 vs 34.6 us, two waves, is a tie).
// Both thresholds are for K x V = 128 x 128.  A smaller state makes a token
// step cheaper, while a chunk keeps its 64 x 64 Gram and inverse, so they
// grow as sqrt(128 * 128 / (K * V)): K = 128, V = 64 crosses over between 32
// and 64 tokens (256 x 32: 310 us per token, 455 chunked; 256 x 64: 572 vs
// 457), K = V = 32 beyond 64 (256 x 64: 182 vs 233 us).
constexpr int64_t kChunkedMinMeanTokens = 32;
constexpr int64_t kChunkedMinMeanTokensOneWave = 16;
constexpr int64_t kComputeUnits = 256;

int64_t chunked_min_mean_tokens(const gdn_config& c, int64_t base) {
    const double kv = static_cast<double>(c.head_k_dim) * c.head_v_dim;
    if (kv >= 128.0 * 128.0) return base;
    return static_cast<int64_t>(std::ceil(base * std::sqrt(128.0 * 128.0 / kv)));
}

bool auto_chunked(const gdn_config& c, bool has_cu, bool has_inter) {
    if (c.kernel_family != GDN_KERNEL_AUTO || has_inter) return false;
    if (c.block_v != 0 || c.block_k != 0 || c.waves_per_group != 0) return false;
    if (c.num_seqs <= 0) return false;
    // the tokens the call processes: without cu_seqlens the rows past
    // num_seqs * tokens_per_seq are not part of any sequence
    const int64_t tokens = has_cu ? c.num_tokens
                                  : static_cast<int64_t>(c.num_seqs) * c.tokens_per_seq;
    if (!has_cu && c.tokens_per_seq <= 1) return false;   // single-token decode
    const bool one_wave = static_cast<int64_t>(c.num_seqs) * c.num_v_heads <= kComputeUnits;
    const int64_t min_mean = chunked_min_mean_tokens(
        c, one_wave ? kChunkedMinMeanTokensOneWave : kChunkedMinMeanTokens);
    if (tokens < min_mean * c.num_seqs) return false;
    gdn::LaunchShape probe{};
    const bool ok = chunked_shape(c, probe) == GDN_OK;
    g_last_error[0] = '\0';
    return ok;
}

// Grid-size check and LDS bytes of a filled-in per-token launch shape.
gdn_status finish_shape(gdn::LaunchShape& s, int V) {
    if (s.groups > INT32_MAX)
        return fail(GDN_ERR_BAD_SHAPE, "grid of %lld workgroups is too large",
                    static_cast<long long>(s.groups));
    s.lds_bytes = gdn::lds_bytes_for(s, V);
    return GDN_OK;
}

// Value-row kernel (VK layout): wavefront units per k-head are G v-heads x
// V/rpw row blocks; the wavefronts never synchronise, so any divisor of the
// unit count may form a workgroup.  Up to 4 wavefronts (MI355X, H 16/32,
// K = V = 128, bf16 state: bs=512 decode 195.1 vs 202.4 us with 8, 256 x 4
// tokens 124.5 vs 134.5 us; fp32 state, 8 long sequences 2.23 vs 3.03 ms),
// except 8 for a single token with fp32 state (bs=512 372.8 vs 380.5 us).
gdn_status value_rows_shape(const gdn_config& c, gdn::LaunchShape& s) {
    const int G = c.num_v_heads / c.num_k_heads;
    const int K = c.head_k_dim, V = c.head_v_dim;
    if (c.kernel_family != GDN_KERNEL_AUTO && c.kernel_family != GDN_KERNEL_VALUE_ROWS)
        return fail(GDN_ERR_BAD_ARGUMENT, "GDN_LAYOUT_VK is served by GDN_KERNEL_VALUE_ROWS only");
    if (c.block_v != 0 || c.block_k != 0)
        return fail(GDN_ERR_BAD_ARGUMENT, "block_v/block_k do not apply to GDN_LAYOUT_VK");
    const int rpw = gdn::vk_rows_per_wave(K, V);
    if (rpw == 0)
        return fail(GDN_ERR_UNSUPPORTED_SHAPE, "no value-row kernel for K = %d, V = %d", K, V);
    const int units = G * (V / rpw);
    if (c.waves_per_group != 0 && units % c.waves_per_group != 0)
        return fail(GDN_ERR_BAD_ARGUMENT, "waves_per_group = %d must divide G*V/%d = %d",
                    c.waves_per_group, rpw, units);
    s.kind = gdn::kKindValueRows;
    s.block_v = rpw;
    s.block_k = K;
    s.rows_rpl_max = 0;
    s.waves = c.waves_per_group ? c.waves_per_group
                                : default_waves(units, c.state_dtype == GDN_DTYPE_BF16 ||
                                                               s.multi_token ? 4 : 8);
    s.groups = static_cast<int64_t>(c.num_seqs) * c.num_k_heads * (units / s.waves);
    return finish_shape(s, V);
}

// Rows per lane (at most 32, 16 or 8) of the row-split kernel for a config
// without a block_k override; 0 if no instance fits.  From same-box runs on
// MI355X (K = V = 128, state streamed from HBM):
//   * one token: 32 from 256 (sequence, k-head) workgroups on, for either
//     storage type.  Against 8 rows per lane, fp32 state: bs=32 24.6 vs
//     27.6 us, bs=64 48.3 vs 50.8 us, bs=512 351 vs 361 us, the 4/8-head
//     shard at bs=256 49.3 vs 53.5 us; bf16 state: bs=64 29.2 vs 31.7 us.
//     Below 256, 8: each head gets its own 8-wavefront workgroup and the
//     state streams through twice as many CUs (bs=1 5.8 vs 7.4 us, bs=8 8.3
//     vs 8.9 us; bf16 state 5.3 vs 7.1 and 6.1 vs 7.6 us);
//   * token loops: 32 from 512 workgroups on (spec verify 264 vs 300 us with
//     8; 64 x 16 tokens 102 vs 135 us), and from 256 when intermediate states
//     are written, with fp32 state or for 8 or more tokens per sequence
//     (16 x 16 tokens: fp32 state 110 vs 119 us, bf16 52 vs 67 us; 24 x 4,
//     fp32, 53.3 vs 59.7 us); 8 otherwise (8 long sequences
//     1.67 vs 2.70 ms with 32; 16 x 4 tokens with intermediates, bf16 state,
//     22.1 vs 22.9 us).
// Other shapes: one token, 32 with fp32 state (bs=64: K = 64, V = 128 25.8
// vs 29.1 us with 8; K = V = 256 184.5 us, where the column tiles take
// 200.8; bs=512 within 3% of the best); with bf16 state 32 below 2048
// workgroups for K, V <= 128 (bs=64, K = 128, V = 64: 15.1 vs 16.8 us with
// 16), else 16 (bs=512: 102.8 vs 107.2 us with 32).  Token loops: 32 at
// K = 256, V = 128 (256 x 16 tokens: 641 vs 900 us with 16); 16 with
// intermediate states and fp32 state where K or V is 64 (256 x 4: 304 vs
// 336 us with 8); else 8.  (Without intermediate states the column tiles
// take those shapes from 1024 workgroups on; see plan_launch.)  A
// waves_per_group override skips instances it cannot form, as does one whose
// single-head workgroup would not fit the LDS budget.
int default_rows_per_lane(const gdn_config& c, const gdn::LaunchShape& s, bool has_inter) {
    const int G = c.num_v_heads / c.num_k_heads;
    const int K = c.head_k_dim, V = c.head_v_dim;
    const bool kv128 = K == 128 && V == 128;
    const bool bf16 = c.state_dtype == GDN_DTYPE_BF16;
    const int64_t groups = static_cast<int64_t>(c.num_seqs) * c.num_k_heads;
    const bool long_inter =
        has_inter && c.num_seqs > 0 &&
        (!bf16 || c.num_tokens >= 8 * static_cast<int64_t>(c.num_seqs));
    const bool wide = s.multi_token ? (groups >= 512 || (long_inter && groups >= 256)) : true;
    int order[3] = {8, 16, 32};
    if (kv128 && !s.multi_token && groups < 256) {
        // fewer than 256 (sequence, k-head) pairs: one head per workgroup
        // and 8 wavefronts each, so the state streams through more CUs
    } else if (kv128 && wide) {
        order[0] = 32; order[1] = 8; order[2] = 16;
    } else if (!s.multi_token && (!bf16 || (groups < 2048 && K <= 128 && V <= 128))) {
        order[0] = 32; order[1] = 16; order[2] = 8;
    } else if (!s.multi_token) {
        order[0] = 16; order[1] = 8; order[2] = 32;
    } else if (K == 256 && V == 128) {
        order[0] = 32; order[1] = 16; order[2] = 8;
    } else if (has_inter && !bf16 && K <= 128 && V <= 128 && !kv128) {
        order[0] = 16; order[1] = 8; order[2] = 32;
    }
    for (int r : order) {
        const int rpw = gdn::rows_per_wave(K, V, r);
        if (rpw == 0) continue;
        const int kw = K / rpw;
        if (c.waves_per_group != 0 &&
            (c.waves_per_group % kw != 0 || G % (c.waves_per_group / kw) != 0))
            continue;
        gdn::LaunchShape one = s;   // one head per workgroup must fit the LDS budget
        one.kind = gdn::kKindRows;
        one.block_k = rpw;
        one.waves = kw;
        if (gdn::lds_bytes_for(one, V) > kMaxDynamicLds) continue;
        return r;
    }
    return 0;
}

// Row-split kernel (KV layout, whole V-column rows per wavefront): rows per
// lane from block_k or the table above, then as many of the k-head's G
// v-heads per workgroup as 8 wavefronts and the LDS budget allow.
gdn_status row_split_shape(const gdn_config& c, bool has_inter, gdn::LaunchShape& s) {
    const int G = c.num_v_heads / c.num_k_heads;
    const int K = c.head_k_dim, V = c.head_v_dim;
    int rpl_max = 0;
    if (c.block_k != 0) {
        for (int r : {16, 8, 32})
            if (gdn::rows_per_wave(K, V, r) == c.block_k) { rpl_max = r; break; }
        if (!rpl_max)
            return fail(GDN_ERR_BAD_ARGUMENT, "no row-split kernel with block_k = %d rows per "
                                              "wavefront for K = %d, V = %d", c.block_k, K, V);
    } else {
        rpl_max = default_rows_per_lane(c, s, has_inter);
        if (!rpl_max)
            return fail(GDN_ERR_BAD_ARGUMENT, "no row-split kernel fits K = %d, V = %d (at most 8 "
                                              "wavefronts per head, %d bytes of LDS, waves_per_group)",
                        K, V, kMaxDynamicLds);
    }
    const int rpw = gdn::rows_per_wave(K, V, rpl_max);
    const int kw = K / rpw;
    s.kind = gdn::kKindRows;
    s.block_v = V;
    s.block_k = rpw;
    s.rows_rpl_max = rpl_max;
    const auto lds_for = [&](int hp) {
        s.waves = hp * kw;
        return gdn::lds_bytes_for(s, V);
    };
    int heads = 0;
    if (c.waves_per_group != 0) {
        if (c.waves_per_group % kw != 0 || G % (c.waves_per_group / kw) != 0)
            return fail(GDN_ERR_BAD_ARGUMENT,
                        "waves_per_group = %d must be a multiple of the %d wavefronts per head "
                        "covering a divisor of G = %d heads", c.waves_per_group, kw, G);
        heads = c.waves_per_group / kw;
        if (lds_for(heads) > kMaxDynamicLds)
            return fail(GDN_ERR_BAD_ARGUMENT, "waves_per_group = %d needs %d bytes of LDS (at most "
                                              "%d)", c.waves_per_group, lds_for(heads), kMaxDynamicLds);
    } else {
        // largest divisor of G within 8 waves and the LDS budget
        for (int hp = G; hp >= 1 && !heads; --hp)
            if (G % hp == 0 && hp * kw <= 8 && lds_for(hp) <= kMaxDynamicLds) heads = hp;
        if (!heads)
            return fail(GDN_ERR_UNSUPPORTED_SHAPE, "no row-split workgroup fits the LDS budget");
    }
    s.waves = heads * kw;
    s.groups = static_cast<int64_t>(c.num_seqs) * c.num_k_heads * (G / heads);
    return finish_shape(s, V);
}

// Token loops at K = V = 128 on fewer than 64 (sequence, k-head) pairs
// (one or a few sequences being verified): 16-column tiles in 2-wavefront
// workgroups spread each head over 8 workgroups, and the dependent token
// chain runs on narrow tiles (1 x 4 tokens with intermediate states, fp32
// state: 8.2 vs 11.2 us; 1 x 8: 11.1 vs 16.4 us; bf16 state 8.1 vs 10.5 us).
bool tiny_token_loop(const gdn_config& c, const gdn::LaunchShape& s) {
    return s.multi_token && c.head_k_dim == 128 && c.head_v_dim == 128 &&
           static_cast<int64_t>(c.num_seqs) * c.num_k_heads < 64;
}

// Column-tile kernel (KV layout, K x block_v tiles per wavefront).
gdn_status column_tiles_shape(const gdn_config& c, gdn::LaunchShape& s) {
    const int G = c.num_v_heads / c.num_k_heads;
    const int K = c.head_k_dim, V = c.head_v_dim;
    if (c.block_k != 0 && c.block_k != K)
        return fail(GDN_ERR_BAD_ARGUMENT, "the column-tile kernel covers all K rows "
                                          "(block_k must be 0 or K = %d)", K);
    if (c.block_v != 0) {
        if (c.block_v != 8 && c.block_v != 16 && c.block_v != 32 && c.block_v != 64)
            return fail(GDN_ERR_BAD_ARGUMENT, "block_v = %d is not 8, 16, 32 or 64", c.block_v);
        if (V % c.block_v != 0)
            return fail(GDN_ERR_BAD_ARGUMENT, "block_v = %d does not divide V = %d", c.block_v, V);
        if (!gdn::instance_exists(K, c.block_v))
            return fail(GDN_ERR_BAD_ARGUMENT, "no kernel for K = %d with block_v = %d", K,
                        c.block_v);
    }
    const bool tiny = c.block_v == 0 && c.waves_per_group == 0 && tiny_token_loop(c, s);
    const int bv = c.block_v ? c.block_v : tiny ? 16 : default_block_v(c);
    const int units = G * (V / bv);
    if (c.waves_per_group != 0 && units % c.waves_per_group != 0)
        return fail(GDN_ERR_BAD_ARGUMENT, "waves_per_group = %d must divide G*V/block_v = %d",
                    c.waves_per_group, units);
    s.kind = gdn::kKindColumns;
    s.block_v = bv;
    s.block_k = K;
    s.rows_rpl_max = 0;
    s.waves = c.waves_per_group ? c.waves_per_group : default_waves(units, tiny ? 2 : 8);
    s.groups = static_cast<int64_t>(c.num_seqs) * c.num_k_heads * (units / s.waves);
    return finish_shape(s, V);
}

// Token loops without intermediate states at K, V <= 128 other than
// K = V = 128, with at least 1024 (sequence, k-head) workgroups: the column
// tiles beat every row split (MI355X, H 16/32: K = 128, V = 64, 256 x 16
// tokens 178.5 vs 182.7 us at 16 rows per lane and 253.6 at 8; K = 64,
// V = 128, 64 x 4 tokens 26.6 vs 31.1 us), within 6% of the best everywhere.
bool prefer_column_tiles(const gdn_config& c, const gdn::LaunchShape& s, bool has_inter) {
    const int K = c.head_k_dim, V = c.head_v_dim;
    if (!s.multi_token || c.block_k != 0 || c.waves_per_group != 0) return false;
    if (tiny_token_loop(c, s)) return true;
    if (has_inter) return false;
    if (K > 128 || V > 128 || (K == 128 && V == 128)) return false;
    return static_cast<int64_t>(c.num_seqs) * c.num_k_heads >= 1024;
}

// Chooses the kernel family, tile and grid of a (size-checked) config, and
// rejects tiling overrides that have no kernel instance.  Calls that the
// chunked kernel does not take default to the row-split kernel (one
// contiguous kilobyte per load/store instruction; measured on MI355X against
// the column tiles: spec verify 264 vs 282 us, the long-varlen batch per
// token 1.67 vs 2.45 ms); calls that override block_v, and shapes without a
// row-split instance, use the column-tile kernel.
gdn_status plan_launch(const gdn_config& c, bool has_cu, bool has_inter, gdn::LaunchShape& s) {
    const int K = c.head_k_dim, V = c.head_v_dim;
    s.K = K;
    s.act = c.act_dtype;
    s.multi_token = (has_cu || c.tokens_per_seq > 1) ? 1 : 0;
    s.chunk = s.multi_token ? gdn::kChunkTokens : 1;
    if (c.kernel_family != GDN_KERNEL_AUTO && c.kernel_family != GDN_KERNEL_COLUMN_TILES &&
        c.kernel_family != GDN_KERNEL_ROW_SPLIT && c.kernel_family != GDN_KERNEL_VALUE_ROWS &&
        c.kernel_family != GDN_KERNEL_CHUNKED)
        return fail(GDN_ERR_BAD_ARGUMENT, "kernel_family = %d is not a GDN_KERNEL_* value",
                    c.kernel_family);
    if (c.waves_per_group < 0 || c.waves_per_group > 8)
        return fail(GDN_ERR_BAD_ARGUMENT, "waves_per_group = %d is not in 0..8", c.waves_per_group);
    if (c.state_layout != GDN_LAYOUT_KV && c.state_layout != GDN_LAYOUT_VK)
        return fail(GDN_ERR_BAD_ARGUMENT, "state_layout = %d is neither GDN_LAYOUT_KV nor _VK",
                    c.state_layout);

    if (c.kernel_family == GDN_KERNEL_CHUNKED || auto_chunked(c, has_cu, has_inter))
        return chunked_shape(c, s);
    if (c.state_layout == GDN_LAYOUT_VK)
        return value_rows_shape(c, s);
    if (c.kernel_family == GDN_KERNEL_VALUE_ROWS)
        return fail(GDN_ERR_BAD_ARGUMENT, "GDN_KERNEL_VALUE_ROWS needs GDN_LAYOUT_VK");
    if (c.kernel_family == GDN_KERNEL_ROW_SPLIT) {
        if (c.block_v != 0 && c.block_v != V)
            return fail(GDN_ERR_BAD_ARGUMENT, "the row-split kernel covers all V columns "
                                              "(block_v must be 0 or V = %d)", V);
        return row_split_shape(c, has_inter, s);
    }
    if (c.kernel_family == GDN_KERNEL_AUTO && c.block_v == 0 &&
        (c.block_k != 0 || (!prefer_column_tiles(c, s, has_inter) &&
                            default_rows_per_lane(c, s, has_inter) > 0)))
        return row_split_shape(c, has_inter, s);
    return column_tiles_shape(c, s);
}

gdn_status check_config(const gdn_config* cfg, bool has_cu, bool has_inter) {
    if (!cfg) return fail(GDN_ERR_NULL_POINTER, "cfg is NULL");
    const gdn_config& c = *cfg;
    if (c.num_seqs < 0) return fail(GDN_ERR_BAD_SHAPE, "num_seqs = %d < 0", c.num_seqs);
    if (c.num_k_heads < 1 || c.num_v_heads < 1)
        return fail(GDN_ERR_BAD_SHAPE, "head counts must be >= 1 (H_k=%d, H_v=%d)", c.num_k_heads,
                    c.num_v_heads);
    if (c.num_v_heads % c.num_k_heads != 0)
        return fail(GDN_ERR_BAD_SHAPE, "H_v=%d is not a multiple of H_k=%d", c.num_v_heads,
                    c.num_k_heads);
    if (!supported_dim(c.head_k_dim) || !supported_dim(c.head_v_dim))
        return fail(GDN_ERR_UNSUPPORTED_SHAPE, "K=%d, V=%d: each must be 32, 64, 128 or 256",
                    c.head_k_dim, c.head_v_dim);
    if (c.act_dtype != GDN_DTYPE_F32 && c.act_dtype != GDN_DTYPE_BF16)
        return fail(GDN_ERR_UNSUPPORTED_DTYPE, "act_dtype %d is neither F32 nor BF16", c.act_dtype);
    if (c.state_dtype != GDN_DTYPE_F32 && c.state_dtype != GDN_DTYPE_BF16)
        return fail(GDN_ERR_UNSUPPORTED_DTYPE, "state_dtype %d is neither F32 nor BF16", c.state_dtype);
    if (c.num_tokens < 0) return fail(GDN_ERR_BAD_SHAPE, "num_tokens < 0");
    if (c.num_tokens > INT32_MAX) return fail(GDN_ERR_BAD_SHAPE, "num_tokens exceeds 2^31-1");
    if (!has_cu) {
        if (c.tokens_per_seq < 1)
            return fail(GDN_ERR_BAD_SHAPE, "tokens_per_seq = %d < 1 without cu_seqlens",
                        c.tokens_per_seq);
        if (static_cast<int64_t>(c.num_seqs) * c.tokens_per_seq > c.num_tokens)
            return fail(GDN_ERR_BAD_SHAPE, "num_seqs*tokens_per_seq = %lld exceeds num_tokens = %lld",
                        static_cast<long long>(c.num_seqs) * c.tokens_per_seq,
                        static_cast<long long>(c.num_tokens));
    }
    if (c.num_slots < 1) return fail(GDN_ERR_BAD_SHAPE, "num_slots must be >= 1");
    if (!std::isfinite(c.scale)) return fail(GDN_ERR_BAD_ARGUMENT, "scale is not finite");
    if (!(c.l2norm_eps >= 0.0f) || !std::isfinite(c.l2norm_eps))
        return fail(GDN_ERR_BAD_ARGUMENT, "l2norm_eps must be finite and >= 0");
    const int64_t qk_dense = static_cast<int64_t>(c.num_k_heads) * c.head_k_dim;
    const int64_t v_dense = static_cast<int64_t>(c.num_v_heads) * c.head_v_dim;
    struct { const char* name; int64_t s; int64_t dense; } strides[] = {
        {"q_stride_tok", c.q_stride_tok, qk_dense},
        {"k_stride_tok", c.k_stride_tok, qk_dense},
        {"v_stride_tok", c.v_stride_tok, v_dense}};
    for (const auto& st : strides) {
        if (st.s == 0) continue;
        if (st.s < st.dense)
            return fail(GDN_ERR_BAD_SHAPE, "%s = %lld is below the dense row size %lld", st.name,
                        static_cast<long long>(st.s), static_cast<long long>(st.dense));
        if (st.s % 8 != 0)
            return fail(GDN_ERR_MISALIGNED, "%s = %lld is not a multiple of 8 elements", st.name,
                        static_cast<long long>(st.s));
    }
    gdn::LaunchShape sh{};
    return plan_launch(c, has_cu, has_inter, sh);
}

gdn_status debug_check_indices(const gdn_config& c, const int32_t* state_idx,
                               const int32_t* cu_seqlens, hipStream_t stream) {
    const int B = c.num_seqs;
    std::vector<int32_t> idx(B), cu(cu_seqlens ? B + 1 : 0);
    if (hipMemcpyAsync(idx.data(), state_idx, sizeof(int32_t) * B, hipMemcpyDeviceToHost, stream) !=
        hipSuccess)
        return fail(GDN_ERR_LAUNCH, "debug checks: copying state_idx failed");
    if (cu_seqlens &&
        hipMemcpyAsync(cu.data(), cu_seqlens, sizeof(int32_t) * (B + 1), hipMemcpyDeviceToHost,
                       stream) != hipSuccess)
        return fail(GDN_ERR_LAUNCH, "debug checks: copying cu_seqlens failed");
    if (hipStreamSynchronize(stream) != hipSuccess)
        return fail(GDN_ERR_LAUNCH, "debug checks: stream synchronisation failed");
    std::vector<char> seen(static_cast<size_t>(c.num_slots), 0);
    for (int i = 0; i < B; ++i) {
        if (idx[i] < 0) continue;
        if (idx[i] >= c.num_slots)
            return fail(GDN_ERR_BAD_ARGUMENT, "state_idx[%d] = %d is not below num_slots = %lld", i,
                        idx[i], static_cast<long long>(c.num_slots));
        if (seen[idx[i]]) return fail(GDN_ERR_BAD_ARGUMENT, "slot %d is used twice", idx[i]);
        seen[idx[i]] = 1;
    }
    if (cu_seqlens) {
        if (cu[0] != 0) return fail(GDN_ERR_BAD_ARGUMENT, "cu_seqlens[0] = %d, not 0", cu[0]);
        for (int i = 0; i < B; ++i)
            if (cu[i + 1] < cu[i])
                return fail(GDN_ERR_BAD_ARGUMENT, "cu_seqlens decreases at %d", i);
        if (cu[B] != c.num_tokens)
            return fail(GDN_ERR_BAD_ARGUMENT, "cu_seqlens[B] = %d differs from num_tokens = %lld",
                        cu[B], static_cast<long long>(c.num_tokens));
    }
    return GDN_OK;
}

// a/b strides: element (t, h) at t*ab_stride_tok + (h/G)*ab_stride_khead + h%G.
gdn_status check_ab_strides(const gdn_config& c) {
    const int G = c.num_v_heads / c.num_k_heads;
    if (c.ab_stride_khead != 0 && c.ab_stride_khead < G)
        return fail(GDN_ERR_BAD_SHAPE, "ab_stride_khead = %d is below G = %d", c.ab_stride_khead, G);
    const int64_t kh = c.ab_stride_khead ? c.ab_stride_khead : G;
    const int64_t row = (c.num_k_heads - 1) * kh + G;
    if (c.ab_stride_tok != 0 && c.ab_stride_tok < row)
        return fail(GDN_ERR_BAD_SHAPE, "ab_stride_tok = %lld is below the %lld elements a token "
                                       "of a/b spans", static_cast<long long>(c.ab_stride_tok),
                    static_cast<long long>(row));
    if (c.ab_stride_tok < 0) return fail(GDN_ERR_BAD_SHAPE, "ab_stride_tok < 0");
    return GDN_OK;
}

// Arguments of the update, with either (a, b, A_log, dt_bias) or precomputed
// (g, beta).
gdn_status validate_update(const void* q, const void* k, const void* v, const void* a, const void* b,
                           const float* A_log, const float* dt_bias, const float* g,
                           const float* beta, const void* state_pool, const int32_t* state_idx,
                           const int32_t* cu_seqlens, const void* out,
                           const void* intermediate_states, const gdn_config* cfg) {
    g_last_error[0] = '\0';
    gdn_status s = check_config(cfg, cu_seqlens != nullptr, intermediate_states != nullptr);
    if (s != GDN_OK) return s;
    s = check_ab_strides(*cfg);
    if (s != GDN_OK) return s;
    // No sequence, or only zero-length ones: nothing is read or written.
    if (cfg->num_seqs == 0 || cfg->num_tokens == 0) return GDN_OK;
    const size_t esize = cfg->act_dtype == GDN_DTYPE_F32 ? 4 : 2;
    const size_t state_align = cfg->state_dtype == GDN_DTYPE_BF16 ? 8 : 16;
    const bool pregated = g != nullptr;
    struct { const void* p; const char* name; size_t align; } ptrs[] = {
        {q, "q", 16}, {k, "k", 16}, {v, "v", 16},
        {pregated ? g : a, pregated ? "g" : "a", pregated ? 4 : esize},
        {pregated ? beta : b, pregated ? "beta" : "b", pregated ? 4 : esize},
        {pregated ? g : A_log, pregated ? "g" : "A_log", 4},
        {pregated ? beta : dt_bias, pregated ? "beta" : "dt_bias", 4},
        {state_pool, "state_pool", state_align}, {state_idx, "state_idx", 4}, {out, "out", 16}};
    for (const auto& e : ptrs) {
        if (!e.p) return fail(GDN_ERR_NULL_POINTER, "%s is NULL", e.name);
        if (!aligned(e.p, e.align))
            return fail(GDN_ERR_MISALIGNED, "%s is not %zu-byte aligned", e.name, e.align);
    }
    if (cu_seqlens && !aligned(cu_seqlens, 4))
        return fail(GDN_ERR_MISALIGNED, "cu_seqlens is not 4-byte aligned");
    if (intermediate_states && cfg->kernel_family == GDN_KERNEL_CHUNKED)
        return fail(GDN_ERR_BAD_ARGUMENT, "the chunked kernel writes no intermediate states");
    if (intermediate_states && !aligned(intermediate_states, state_align))
        return fail(GDN_ERR_MISALIGNED, "intermediate_states is not %zu-byte aligned", state_align);
    return GDN_OK;
}

// Bytes of the two-kernel chunked form's workspace (0 for no work).
size_t chunk_workspace_bytes(const gdn_config& c) {
    if (c.num_seqs <= 0 || c.num_tokens <= 0 || c.num_v_heads < 1) return 0;
    return static_cast<size_t>(gdn::chunk_ws_slots(c.num_tokens, c.num_seqs)) *
           static_cast<size_t>(c.num_v_heads) * static_cast<size_t>(gdn::chunk_ws_entry_bytes());
}

// workspace (chunked family only): NULL runs the one-kernel form; otherwise
// at least chunk_workspace_bytes(cfg), 256-byte aligned.
gdn_status run_update(const void* q, const void* k, const void* v, const void* a, const void* b,
                      const float* A_log, const float* dt_bias, const float* g, const float* beta,
                      void* state_pool, const int32_t* state_idx, const int32_t* cu_seqlens,
                      void* out, void* intermediate_states, const gdn_config* cfg, void* stream,
                      void* workspace = nullptr, size_t workspace_bytes = 0) {
    gdn_status s = validate_update(q, k, v, a, b, A_log, dt_bias, g, beta, state_pool, state_idx,
                                   cu_seqlens, out, intermediate_states, cfg);
    if (s != GDN_OK) return s;
    const gdn_config& c = *cfg;
    if (workspace) {
        if (!aligned(workspace, 256))
            return fail(GDN_ERR_MISALIGNED, "workspace is not 256-byte aligned");
        if (workspace_bytes < chunk_workspace_bytes(c))
            return fail(GDN_ERR_BAD_ARGUMENT, "workspace holds %zu bytes; this call needs %zu",
                        workspace_bytes, chunk_workspace_bytes(c));
    }
    if (c.num_seqs == 0 || c.num_tokens == 0) return GDN_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (c.flags & GDN_FLAG_DEBUG_CHECKS) {
        s = debug_check_indices(c, state_idx, cu_seqlens, st);
        if (s != GDN_OK) return s;
    }
    const bool has_cu = cu_seqlens != nullptr;
    gdn::LaunchShape sh{};
    s = plan_launch(c, has_cu, intermediate_states != nullptr, sh);
    if (s != GDN_OK) return s;

    gdn::FusedParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.a = a;
    p.b = b;
    p.g = g;
    p.beta = beta;
    p.A_log = A_log;
    p.dt_bias = dt_bias;
    p.pool = state_pool;
    p.state_idx = state_idx;
    p.cu_seqlens = cu_seqlens;
    p.out = out;
    p.inter = intermediate_states;
    const int G = c.num_v_heads / c.num_k_heads;
    const int64_t qk_dense = static_cast<int64_t>(c.num_k_heads) * c.head_k_dim;
    p.q_stride = c.q_stride_tok ? c.q_stride_tok : qk_dense;
    p.k_stride = c.k_stride_tok ? c.k_stride_tok : qk_dense;
    p.v_stride = c.v_stride_tok ? c.v_stride_tok : static_cast<int64_t>(c.num_v_heads) * c.head_v_dim;
    p.ab_stride = c.ab_stride_tok ? c.ab_stride_tok : c.num_v_heads;
    p.ab_khead = c.ab_stride_khead ? c.ab_stride_khead : G;
    p.T = has_cu ? 0 : c.tokens_per_seq;
    p.Hk = c.num_k_heads;
    p.Hv = c.num_v_heads;
    p.G = G;
    p.V = c.head_v_dim;
    p.groups_per_khead =
        static_cast<int32_t>(sh.groups / (static_cast<int64_t>(c.num_seqs) * c.num_k_heads));
    p.scale = c.scale > 0.0f ? c.scale : 1.0f / std::sqrt(static_cast<float>(c.head_k_dim));
    p.eps = c.l2norm_eps;
    p.write_final = (c.flags & GDN_FLAG_NO_FINAL_WRITEBACK) ? 0 : 1;
    p.state_bf16 = c.state_dtype == GDN_DTYPE_BF16 ? 1 : 0;
    p.state_vk = c.state_layout == GDN_LAYOUT_VK ? 1 : 0;

    static const bool log = [] {
        const char* e = std::getenv("GDN_LOG");
        return e && e[0] == '1';
    }();
    if (log)
        std::fprintf(stderr,
                     "[gdn] %s K=%d V=%d act=%s state=%s gates=%s multi_token=%d block_v=%d block_k=%d "
                     "waves=%d chunk=%d groups=%lld lds=%d\n",
                     sh.kind == gdn::kKindRows        ? "rows"
                     : sh.kind == gdn::kKindValueRows ? "value-rows"
                     : sh.kind == gdn::kKindChunked   ? (workspace ? "chunked (prep + state pass)"
                                                                   : "chunked")
                                                      : "columns",
                     sh.K, c.head_v_dim, sh.act ? "bf16" : "f32", p.state_bf16 ? "bf16" : "f32",
                     g ? "precomputed" : "fused",
                     sh.multi_token, sh.block_v, sh.block_k, sh.waves, sh.chunk,
                     static_cast<long long>(sh.groups), sh.lds_bytes);

    const hipError_t e =
        sh.kind != gdn::kKindChunked ? gdn::launch_fused(sh, p, st)
        : workspace ? gdn::launch_chunked_ws(sh, p, c.num_seqs, c.num_tokens, workspace, st)
                    : gdn::launch_chunked(sh, p, st);
    if (e != hipSuccess)
        return fail(GDN_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
    return GDN_OK;
}

}  // namespace

extern "C" {

void gdn_default_config(gdn_config* cfg) {
    if (!cfg) return;
    std::memset(cfg, 0, sizeof(*cfg));
    cfg->tokens_per_seq = 1;
    cfg->act_dtype = GDN_DTYPE_F32;
    cfg->scale = 0.0f;
    cfg->l2norm_eps = 1e-6f;
}

gdn_status gdn_validate(const void* q, const void* k, const void* v, const void* a, const void* b,
                        const float* A_log, const float* dt_bias, const void* state_pool,
                        const int32_t* state_idx, const int32_t* cu_seqlens, const void* out,
                        const void* intermediate_states, const gdn_config* cfg) {
    return validate_update(q, k, v, a, b, A_log, dt_bias, nullptr, nullptr, state_pool, state_idx,
                           cu_seqlens, out, intermediate_states, cfg);
}

gdn_status gdn_plan(const gdn_config* cfg, int has_cu_seqlens, int has_intermediate_states,
                    gdn_launch_info* info) {
    g_last_error[0] = '\0';
    if (!info) return fail(GDN_ERR_NULL_POINTER, "info is NULL");
    gdn_status s = check_config(cfg, has_cu_seqlens != 0, has_intermediate_states != 0);
    if (s != GDN_OK) return s;
    gdn::LaunchShape sh{};
    s = plan_launch(*cfg, has_cu_seqlens != 0, has_intermediate_states != 0, sh);
    if (s != GDN_OK) return s;
    info->kernel_family = sh.kind == gdn::kKindRows        ? GDN_KERNEL_ROW_SPLIT
                          : sh.kind == gdn::kKindValueRows ? GDN_KERNEL_VALUE_ROWS
                          : sh.kind == gdn::kKindChunked   ? GDN_KERNEL_CHUNKED
                                                           : GDN_KERNEL_COLUMN_TILES;
    info->block_k = sh.block_k;
    info->block_v = sh.block_v;
    info->waves_per_group = sh.waves;
    info->tokens_per_chunk = sh.chunk;
    info->multi_token = sh.multi_token;
    info->workgroups = sh.groups;
    info->threads_per_group = sh.waves * 64;
    info->lds_bytes = sh.lds_bytes;
    return GDN_OK;
}

gdn_status gdn_gating_delta_rule_update(const void* q, const void* k, const void* v, const void* a,
                                        const void* b, const float* A_log, const float* dt_bias,
                                        void* state_pool, const int32_t* state_idx,
                                        const int32_t* cu_seqlens, void* out,
                                        void* intermediate_states, const gdn_config* cfg,
                                        void* stream) {
    return run_update(q, k, v, a, b, A_log, dt_bias, nullptr, nullptr, state_pool, state_idx,
                      cu_seqlens, out, intermediate_states, cfg, stream);
}

gdn_status gdn_chunk_gated_delta_rule_fwd(const void* q, const void* k, const void* v,
                                          const void* a, const void* b, const float* A_log,
                                          const float* dt_bias, void* state_pool,
                                          const int32_t* state_idx, const int32_t* cu_seqlens,
                                          void* out, void* workspace, size_t workspace_bytes,
                                          const gdn_config* cfg, void* stream) {
    g_last_error[0] = '\0';
    if (!cfg) return fail(GDN_ERR_NULL_POINTER, "cfg is NULL");
    if (cfg->kernel_family != GDN_KERNEL_AUTO && cfg->kernel_family != GDN_KERNEL_CHUNKED)
        return fail(GDN_ERR_BAD_ARGUMENT, "kernel_family = %d: the chunked forward runs "
                                          "GDN_KERNEL_CHUNKED only", cfg->kernel_family);
    gdn_config c = *cfg;
    c.kernel_family = GDN_KERNEL_CHUNKED;
    return run_update(q, k, v, a, b, A_log, dt_bias, nullptr, nullptr, state_pool, state_idx,
                      cu_seqlens, out, nullptr, &c, stream, workspace, workspace_bytes);
}

size_t gdn_chunk_workspace_bytes(const gdn_config* cfg) {
    return cfg ? chunk_workspace_bytes(*cfg) : 0;
}

gdn_status gdn_chunk_gated_delta_rule_fwd_noalloc(const void* q, const void* k, const void* v,
                                                  const void* a, const void* b, const float* A_log,
                                                  const float* dt_bias, void* state_pool,
                                                  const int32_t* state_idx,
                                                  const int32_t* cu_seqlens, void* out,
                                                  const gdn_config* cfg, void* stream) {
    g_last_error[0] = '\0';
    if (!cfg) return fail(GDN_ERR_NULL_POINTER, "cfg is NULL");
    if (cfg->kernel_family != GDN_KERNEL_AUTO && cfg->kernel_family != GDN_KERNEL_CHUNKED)
        return fail(GDN_ERR_BAD_ARGUMENT, "kernel_family = %d: the chunked forward runs "
                                          "GDN_KERNEL_CHUNKED only", cfg->kernel_family);
    gdn_config c = *cfg;
    c.kernel_family = GDN_KERNEL_CHUNKED;
    gdn_status s = validate_update(q, k, v, a, b, A_log, dt_bias, nullptr, nullptr, state_pool,
                                   state_idx, cu_seqlens, out, nullptr, &c);
    if (s != GDN_OK) return s;
    const size_t need = chunk_workspace_bytes(c);
    if (need > gdn::scratch_bytes())
        return fail(GDN_ERR_BAD_ARGUMENT, "this call needs %zu bytes of scratch; the library's "
                                          "fixed scratch holds %zu (GDN_CHUNK_SCRATCH_BYTES): pass "
                                          "a workspace to gdn_chunk_gated_delta_rule_fwd instead",
                    need, gdn::scratch_bytes());
    if (need == 0) return GDN_OK;   // no sequence or no token: nothing to do
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = -1;
    hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(GDN_ERR_LAUNCH, "cannot tell the stream's device: %s", hipGetErrorString(e));
    void* ws = nullptr;
    e = gdn::scratch_address(dev, &ws);
    if (e != hipSuccess)
        return fail(GDN_ERR_LAUNCH, "looking up the device scratch failed: %s", hipGetErrorString(e));
    return run_update(q, k, v, a, b, A_log, dt_bias, nullptr, nullptr, state_pool, state_idx,
                      cu_seqlens, out, nullptr, &c, stream, ws, gdn::scratch_bytes());
}

gdn_status gdn_recurrent_update(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, void* state_pool, const int32_t* state_idx,
                                const int32_t* cu_seqlens, void* out, void* intermediate_states,
                                const gdn_config* cfg, void* stream) {
    g_last_error[0] = '\0';
    if (!g || !beta) {
        if (cfg && (cfg->num_seqs == 0 || cfg->num_tokens == 0)) return GDN_OK;
        return fail(GDN_ERR_NULL_POINTER, "g and beta must not be NULL");
    }
    return run_update(q, k, v, nullptr, nullptr, nullptr, nullptr, g, beta, state_pool, state_idx,
                      cu_seqlens, out, intermediate_states, cfg, stream);
}

gdn_status gdn_gating(const void* a, const void* b, const float* A_log, const float* dt_bias,
                      float* g, float* beta, const gdn_config* cfg, void* stream) {
    g_last_error[0] = '\0';
    if (!cfg) return fail(GDN_ERR_NULL_POINTER, "cfg is NULL");
    const gdn_config& c = *cfg;
    if (c.state_dtype != GDN_DTYPE_F32 && c.state_dtype != GDN_DTYPE_BF16)
        return fail(GDN_ERR_UNSUPPORTED_DTYPE, "state_dtype %d is neither F32 nor BF16", c.state_dtype);
    if (c.num_tokens < 0) return fail(GDN_ERR_BAD_SHAPE, "num_tokens < 0");
    if (c.num_k_heads < 1 || c.num_v_heads < 1 || c.num_v_heads % c.num_k_heads != 0)
        return fail(GDN_ERR_BAD_SHAPE, "H_v = %d must be a positive multiple of H_k = %d",
                    c.num_v_heads, c.num_k_heads);
    if (c.act_dtype != GDN_DTYPE_F32 && c.act_dtype != GDN_DTYPE_BF16)
        return fail(GDN_ERR_UNSUPPORTED_DTYPE, "act_dtype %d is neither F32 nor BF16", c.act_dtype);
    gdn_status s = check_ab_strides(c);
    if (s != GDN_OK) return s;
    if (c.num_tokens == 0) return GDN_OK;
    const size_t esize = c.act_dtype == GDN_DTYPE_F32 ? 4 : 2;
    struct { const void* p; const char* name; size_t align; } ptrs[] = {
        {a, "a", esize}, {b, "b", esize}, {A_log, "A_log", 4}, {dt_bias, "dt_bias", 4},
        {g, "g", 4}, {beta, "beta", 4}};
    for (const auto& e : ptrs) {
        if (!e.p) return fail(GDN_ERR_NULL_POINTER, "%s is NULL", e.name);
        if (!aligned(e.p, e.align))
            return fail(GDN_ERR_MISALIGNED, "%s is not %zu-byte aligned", e.name, e.align);
    }
    const int G = c.num_v_heads / c.num_k_heads;
    const hipError_t e = gdn::launch_gating(
        a, b, A_log, dt_bias, g, beta, c.num_tokens * c.num_v_heads, c.num_v_heads, G,
        c.ab_stride_tok ? c.ab_stride_tok : c.num_v_heads, c.ab_stride_khead ? c.ab_stride_khead : G,
        c.act_dtype, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "gating launch failed: %s", hipGetErrorString(e));
    return GDN_OK;
}

const char* gdn_status_string(int status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL_POINTER: return "a required pointer is NULL";
        case GDN_ERR_BAD_SHAPE: return "inconsistent or invalid sizes";
        case GDN_ERR_UNSUPPORTED_SHAPE: return "unsupported head dimension";
        case GDN_ERR_UNSUPPORTED_DTYPE: return "unsupported activation dtype";
        case GDN_ERR_MISALIGNED: return "pointer or stride misaligned";
        case GDN_ERR_LAUNCH: return "kernel launch failed";
        case GDN_ERR_BAD_ARGUMENT: return "invalid argument";
    }
    return "unknown status";
}

const char* gdn_last_error_message(void) { return g_last_error; }

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

}  // extern "C"
