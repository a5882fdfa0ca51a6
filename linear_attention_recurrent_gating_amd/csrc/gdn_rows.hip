// Row-split kernels of the fused sigmoid gating + gated delta-rule update
// (KV state layout) for gfx950: a wavefront holds whole V-column rows of the
// state, so every 128-bit load or store instruction moves one contiguous
// kilobyte of the tile.  The operation is the fused kernel of vLLM PR #35777
// (implementation section); sglang PR #18271 (Benchmarking and Profiling)
// shows the same kernel gaining from fuller tiles, which whole rows carry to
// the limit.

#include "gdn_tile.h"

namespace gdn {
namespace {

// Layout shared by both kernels.  LPR = V/4 lanes cover one V-column row, so
// each 128-bit load or store instruction of a wave moves RG = 64/LPR
// consecutive rows: one contiguous kilobyte of the tile.  Lane l
// holds columns 4*(l % LPR)..+3 of rows kw*RPW + RG*i + l/LPR (i < RPL); the
// K rows of a head are split over KW wavefronts.  S^T k, S^T q and k.q are
// reduced in-lane, across the wave's row groups with permlane swaps, and
// across the KW wavefronts of the head through LDS, summed in a fixed order
// so every wave derives the same u.
template <int K, int V, int RPL_MAX>
struct RowSplit {
    static constexpr int LPR = V / 4;                                   // lanes per row
    static constexpr int RG = kWave / LPR;                              // rows per instruction
    static constexpr int RPL = (K / RG < RPL_MAX) ? K / RG : RPL_MAX;   // rows per lane
    static constexpr int RPW = RPL * RG;                                // rows per wave
    static constexpr int KW = K / RPW;                                  // waves per head
    static constexpr int PART = 2 * V + 4;                              // partial sums per wave
};

// One token's partial sums of a wavefront, written to its LDS block `mine`
// ([PART] floats: S^T k, S^T q, k.q): in-lane over the RPL rows, then across
// the wave's row groups (every lane of a column then holds the same sum).
template <int RPL, int LPR, int V>
__device__ __forceinline__ void rows_partials(const float4 (&S)[RPL], const float (&kh)[RPL],
                                              const float (&qh)[RPL], float* mine, int col,
                                              bool writer, bool kq_writer) {
    float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f}, kq = 0.f;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        const float s4[4] = {S[i].x, S[i].y, S[i].z, S[i].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            pk[c] = __builtin_fmaf(s4[c], kh[i], pk[c]);
            pq[c] = __builtin_fmaf(s4[c], qh[i], pq[c]);
        }
        kq = __builtin_fmaf(kh[i], qh[i], kq);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        pk[c] = sum_row_groups<LPR>(pk[c]);
        pq[c] = sum_row_groups<LPR>(pq[c]);
    }
    kq = sum_row_groups<LPR>(kq);
    if (writer) {
        *reinterpret_cast<float4*>(mine + col) = make_float4(pk[0], pk[1], pk[2], pk[3]);
        *reinterpret_cast<float4*>(mine + V + col) = make_float4(pq[0], pq[1], pq[2], pq[3]);
        if (kq_writer) mine[2 * V] = kq;
    }
}

// After the barrier: sums the KW partial blocks of the head in a fixed order,
// forms u = beta*(v - gamma*S^T k) and o = gamma*S^T q + u*(k.q) for this
// lane's four columns, applies the decay and rank-1 update to the lane's
// rows, and returns o.
template <int RPL, int KW, int V>
__device__ __forceinline__ float4 rows_token_update(float4 (&S)[RPL], const float (&kh)[RPL],
                                                    const float* head_part, int col, float4 vv,
                                                    float gamma, float beta) {
    constexpr int PART = 2 * V + 4;
    float4 PK = make_float4(0.f, 0.f, 0.f, 0.f), PQ = PK;
    float KQ = 0.f;
#pragma unroll
    for (int w = 0; w < KW; ++w) {
        const float4 a4 = *reinterpret_cast<const float4*>(head_part + w * PART + col);
        const float4 b4 = *reinterpret_cast<const float4*>(head_part + w * PART + V + col);
        PK.x += a4.x; PK.y += a4.y; PK.z += a4.z; PK.w += a4.w;
        PQ.x += b4.x; PQ.y += b4.y; PQ.z += b4.z; PQ.w += b4.w;
        KQ += head_part[w * PART + 2 * V];
    }
    float4 u, o;
    u.x = beta * (vv.x - gamma * PK.x);
    u.y = beta * (vv.y - gamma * PK.y);
    u.z = beta * (vv.z - gamma * PK.z);
    u.w = beta * (vv.w - gamma * PK.w);
    o.x = __builtin_fmaf(u.x, KQ, gamma * PQ.x);
    o.y = __builtin_fmaf(u.y, KQ, gamma * PQ.y);
    o.z = __builtin_fmaf(u.z, KQ, gamma * PQ.z);
    o.w = __builtin_fmaf(u.w, KQ, gamma * PQ.w);
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        S[i].x = __builtin_fmaf(kh[i], u.x, gamma * S[i].x);
        S[i].y = __builtin_fmaf(kh[i], u.y, gamma * S[i].y);
        S[i].z = __builtin_fmaf(kh[i], u.z, gamma * S[i].z);
        S[i].w = __builtin_fmaf(kh[i], u.w, gamma * S[i].w);
    }
    return o;
}

// The single token's q and k for the row-split kernel, in two halves so the
// raw loads can be issued ahead of the state loads: DPP rows 0 and 1 of
// wavefront 0 hold q and k, K/16 elements per lane.
template <int K, int ACT>
struct SingleTokenQK {
    static constexpr int EPL = K / 16;
    float x[EPL];
    bool active, is_k;

    __device__ __forceinline__ void load(const FusedParams& p, int j, int64_t t, int wave,
                                         int lane) {
        const int vec = wave * 4 + lane / 16;
        active = vec < 2;
        is_k = vec == 1;
        if (active) {
            const int lr = lane % 16;
            if (is_k)
                load_act<ACT, EPL>(p.k, t * p.k_stride + static_cast<int64_t>(j) * K + lr * EPL, x);
            else
                load_act<ACT, EPL>(p.q, t * p.q_stride + static_cast<int64_t>(j) * K + lr * EPL, x);
        }
    }

    // Same arithmetic, in the same order, as stage_qk.
    template <typename POS>
    __device__ __forceinline__ void finish(const FusedParams& p, float* qs, float* ks, int lane,
                                           POS pos) {
        if (!active) return;
        const int lr = lane % 16;
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
        ss = sum_dpp_row(ss);
        const float f = (is_k ? 1.0f : p.scale) * rsqrtf(ss + p.eps);
        float* dst = is_k ? ks : qs;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dst[pos(lr * EPL + e)] = x[e] * f;
    }
};

// Single token per sequence (decode).  The small loads (q, k, gates, v) are
// issued before the state tile, and q/k are normalised into LDS while the
// tile streams in.
template <int K, int V, int ACT, int RPL_MAX>
__global__ void __launch_bounds__(kMaxThreads)
gdn_decode_rows(const FusedParams p) {
    using L = RowSplit<K, V, RPL_MAX>;
    constexpr int LPR = L::LPR, RG = L::RG, RPL = L::RPL, RPW = L::RPW, KW = L::KW;
    static_assert(LPR >= 8 && RPL >= 1 && K % RPW == 0, "unsupported K/V pair");

    extern __shared__ __align__(16) float lds[];
    float* qs = lds;              // [K] normalised q, permuted
    float* ks = lds + K;          // [K] normalised k, permuted
    float* part = lds + 2 * K;    // [heads in group][KW][PART] partial sums

    const int waves = blockDim.x / kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;

    int64_t blk = blockIdx.x;
    const int gslice = static_cast<int>(blk % p.groups_per_khead);
    blk /= p.groups_per_khead;
    const int j = static_cast<int>(blk % p.Hk);
    const int seq = static_cast<int>(blk / p.Hk);

    const int32_t slot = p.state_idx[seq];
    if (slot < 0) return;                         // padded: touch nothing
    const int64_t t = static_cast<int64_t>(seq);  // one token per sequence

    const int heads_per_group = waves / KW;
    const int hl = wave / KW;                     // head within the workgroup
    const int kw = wave % KW;                     // row block of the head
    const int h = j * p.G + gslice * heads_per_group + hl;
    const int col = 4 * (lane % LPR);
    const int rg = lane / LPR;

    // Small loads first (q/k for the staging rows, gates, v): they return
    // while the state tile is still streaming in.
    SingleTokenQK<K, ACT> qk;
    qk.load(p, j, t, wave, lane);
    float gamma, beta;
    token_gates<ACT>(p, t, h, gamma, beta);
    float vv[4];
    load_act<ACT, 4>(p.v, t * p.v_stride + static_cast<int64_t>(h) * V + col, vv);

    constexpr uint32_t row_step = RG * V;   // one kilobyte of fp32 state
    const uint32_t lane_elem = static_cast<uint32_t>((kw * RPW + rg) * V + col);
    const TileIO tio = tile_io(p.pool, p.state_bf16, static_cast<size_t>(slot) * p.Hv + h, K * V, lane_elem);

    const auto rows_at = [](int i) { return static_cast<uint32_t>(i) * row_step; };
    u32x4 raw[RPL];
    tile_issue<RPL>(tio, rows_at, raw);

    // rows kw*RPW + RG*i + rg of the head sit at kw*RPW + rg*RPL + i
    qk.finish(p, qs, ks, lane, [](int kappa) {
        const int r = kappa % RPW;
        return (kappa - r) + (r % RG) * RPL + r / RG;
    });
    lds_barrier();

    float kh[RPL], qh[RPL];
    lds_read<RPL>(ks + kw * RPW + rg * RPL, kh);
    lds_read<RPL>(qs + kw * RPW + rg * RPL, qh);
    float4 S[RPL];
    tile_unpack<RPL>(tio.bf16, raw, S);
    rows_partials<RPL, LPR, V>(S, kh, qh, part + (hl * KW + kw) * L::PART, col, rg == 0, lane == 0);
    lds_barrier();
    const float4 o = rows_token_update<RPL, KW, V>(S, kh, part + hl * KW * L::PART, col,
                                                   make_float4(vv[0], vv[1], vv[2], vv[3]), gamma, beta);
    if (kw == 0 && rg == 0) store4_act<ACT>(p.out, (t * p.Hv + h) * static_cast<int64_t>(V) + col, o);
    if (p.inter) {
        const TileIO it = tile_io(p.inter, p.state_bf16, static_cast<size_t>(t) * p.Hv + h, K * V, lane_elem);
        tile_store_all<RPL>(it, rows_at, S);
    }
    if (p.write_final) tile_store_all<RPL>(tio, rows_at, S);
}

// Row split over a token loop (T tokens per sequence, or cu_seqlens).  The
// KW wavefronts of a head keep their rows of the state in VGPRs for the whole
// sequence.  Per token they meet once in LDS: the partial-sum blocks are
// double-buffered by token parity, so one barrier per token suffices (a wave
// that writes the block of token t+2 has passed the barrier of token t+1,
// which every wave reaches only after reading the blocks of token t).  Chunks
// of CHUNK tokens of normalised q/k (shared by the workgroup), of v (per
// head) and of the gates (one token per lane) are staged in LDS.  Per token
// the arithmetic, and its order, is the single-token kernel's, so a T-token
// call equals T chained single-token calls bit for bit.
template <int K, int V, int ACT, int RPL_MAX, int CHUNK>
__global__ void __launch_bounds__(kMaxThreads)
gdn_rows_tokens(const FusedParams p) {
    using L = RowSplit<K, V, RPL_MAX>;
    constexpr int LPR = L::LPR, RG = L::RG, RPL = L::RPL, RPW = L::RPW, KW = L::KW;
    static_assert(LPR >= 8 && RPL >= 1 && K % RPW == 0, "unsupported K/V pair");
    static_assert(CHUNK >= 1 && CHUNK <= kWave, "one gate lane per staged token");

    extern __shared__ __align__(16) float lds[];
    const int waves = blockDim.x / kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int heads_per_group = waves / KW;
    float* qs = lds;                                   // [CHUNK][K] normalised q, permuted
    float* ks = lds + CHUNK * K;                       // [CHUNK][K] normalised k, permuted
    float* vs = lds + 2 * CHUNK * K;                   // [heads][CHUNK][V]
    float* part = vs + heads_per_group * CHUNK * V;    // [2][heads][KW][PART]

    int64_t blk = blockIdx.x;
    const int gslice = static_cast<int>(blk % p.groups_per_khead);
    blk /= p.groups_per_khead;
    const int j = static_cast<int>(blk % p.Hk);
    const int seq = static_cast<int>(blk / p.Hk);

    const int32_t slot = p.state_idx[seq];
    int64_t t0, t1;
    if (p.cu_seqlens) {
        t0 = p.cu_seqlens[seq];
        t1 = p.cu_seqlens[seq + 1];
    } else {
        t0 = static_cast<int64_t>(seq) * p.T;
        t1 = t0 + p.T;
    }
    if (slot < 0 || t1 <= t0) return;  // padded or empty: touch nothing

    const int hl = wave / KW;                     // head within the workgroup
    const int kw = wave % KW;                     // row block of the head
    const int h = j * p.G + gslice * heads_per_group + hl;
    const int col = 4 * (lane % LPR);
    const int rg = lane / LPR;

    constexpr uint32_t row_step = RG * V;
    const uint32_t lane_elem = static_cast<uint32_t>((kw * RPW + rg) * V + col);
    const TileIO tio = tile_io(p.pool, p.state_bf16, static_cast<size_t>(slot) * p.Hv + h, K * V, lane_elem);
    const auto rows_at = [](int i) { return static_cast<uint32_t>(i) * row_step; };
    u32x4 raw[RPL];
    tile_issue<RPL>(tio, rows_at, raw);
    float4 S[RPL];

    float* hv = vs + hl * (CHUNK * V);            // this head's staged v rows
    float gam, bet;                               // lane tau: token tau's gates
    const auto stage = [&](int64_t c0, int nt) {
        // rows kw*RPW + RG*i + rg of the head sit at kw*RPW + rg*RPL + i
        stage_qk<K, ACT>(p, qs, ks, j, c0, nt, wave, waves, lane, [](int kappa) {
            const int r = kappa % RPW;
            return (kappa - r) + (r % RG) * RPL + r / RG;
        });
        gam = 1.0f;
        bet = 0.0f;
        if (lane < nt) token_gates<ACT>(p, c0 + lane, h, gam, bet);
        // the KW wavefronts of the head stage its v rows, RG tokens per pass each
        for (int tok = kw * RG + rg; tok < nt; tok += KW * RG) {
            float vv[4];
            load_act<ACT, 4>(p.v, (c0 + tok) * p.v_stride + static_cast<int64_t>(h) * V + col, vv);
            *reinterpret_cast<float4*>(hv + tok * V + col) = make_float4(vv[0], vv[1], vv[2], vv[3]);
        }
        lds_barrier();
    };

    // Rotated loop: the first chunk is staged while the state loads are in
    // flight, and the raw state words die at the unpack.
    int64_t c0 = t0;
    int nt = static_cast<int>(t1 - c0 < CHUNK ? t1 - c0 : CHUNK);
    stage(c0, nt);
    tile_unpack<RPL>(tio.bf16, raw, S);
    for (;;) {
        for (int tau = 0; tau < nt; ++tau) {
            const int64_t t = c0 + tau;
            const float gamma = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gam), tau));
            const float beta = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bet), tau));
            float kh[RPL], qh[RPL];
            lds_read<RPL>(ks + tau * K + kw * RPW + rg * RPL, kh);
            lds_read<RPL>(qs + tau * K + kw * RPW + rg * RPL, qh);
            float* buf = part + static_cast<int>((t - t0) & 1) * (waves * L::PART);
            rows_partials<RPL, LPR, V>(S, kh, qh, buf + (hl * KW + kw) * L::PART, col, rg == 0, lane == 0);
            lds_barrier();
            const float4 vv = *reinterpret_cast<const float4*>(hv + tau * V + col);
            const float4 o = rows_token_update<RPL, KW, V>(S, kh, buf + hl * KW * L::PART, col, vv,
                                                           gamma, beta);
            if (kw == 0 && rg == 0)
                store4_act<ACT>(p.out, (t * p.Hv + h) * static_cast<int64_t>(V) + col, o);
            if (p.inter) {
                const TileIO it =
                    tile_io(p.inter, p.state_bf16, static_cast<size_t>(t) * p.Hv + h, K * V, lane_elem);
                tile_store_all<RPL>(it, rows_at, S);
            }
        }
        c0 += CHUNK;
        if (c0 >= t1) break;
        nt = static_cast<int>(t1 - c0 < CHUNK ? t1 - c0 : CHUNK);
        lds_barrier();   // the next chunk reuses the staged rows
        stage(c0, nt);
    }
    if (p.write_final) tile_store_all<RPL>(tio, rows_at, S);
}

// ------------------------------------------------------------ instance table

// Row-split instances: RPL_MAX 32 (128 state VGPRs per lane), 16 (64) and
// 8 (32), while a head needs at most 8 wavefronts.
template <int K, int V, int ACT, int RPLM>
KernelFn pick_rows(int multi) {
    if constexpr (RowSplit<K, V, RPLM>::KW <= 8)
        return multi ? &gdn_rows_tokens<K, V, ACT, RPLM, kChunkTokens> : &gdn_decode_rows<K, V, ACT, RPLM>;
    else return nullptr;
}

template <int K, int V, int ACT>
KernelFn rows_by_rpl(int rpl, int multi) {
    return rpl == 8    ? pick_rows<K, V, ACT, 8>(multi)
           : rpl == 16 ? pick_rows<K, V, ACT, 16>(multi)
           : rpl == 32 ? pick_rows<K, V, ACT, 32>(multi)
                       : nullptr;
}

template <int K, int ACT>
KernelFn rows_by_v(int V, int rpl, int multi) {
    switch (V) {
        case 32: return rows_by_rpl<K, 32, ACT>(rpl, multi);
        case 64: return rows_by_rpl<K, 64, ACT>(rpl, multi);
        case 128: return rows_by_rpl<K, 128, ACT>(rpl, multi);
        case 256: return rows_by_rpl<K, 256, ACT>(rpl, multi);
        default: return nullptr;
    }
}

template <int ACT>
KernelFn rows_by_k(int K, int V, int rpl, int multi) {
    switch (K) {
        case 32: return rows_by_v<32, ACT>(V, rpl, multi);
        case 64: return rows_by_v<64, ACT>(V, rpl, multi);
        case 128: return rows_by_v<128, ACT>(V, rpl, multi);
        case 256: return rows_by_v<256, ACT>(V, rpl, multi);
        default: return nullptr;
    }
}

}  // namespace

KernelFn select_rows(int K, int V, int act, int rpl, int multi) {
    return act == 0 ? rows_by_k<0>(K, V, rpl, multi) : rows_by_k<1>(K, V, rpl, multi);
}

int rows_per_wave(int K, int V, int rpl_max) {
    if (!select_rows(K, V, 0, rpl_max, 0)) return 0;
    const int rg = kWave / (V / 4);
    const int rpl = K / rg < rpl_max ? K / rg : rpl_max;
    return rpl * rg;
}

}  // namespace gdn
