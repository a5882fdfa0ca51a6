// Fused sigmoid gating + gated delta-rule state update for gfx950 (CDNA4).
//
// The operation is the fused decode kernel described by vLLM PR #35777
// (implementation section: gating folded into the recurrent delta-rule update,
// rsqrt normalisation, a speculative-decoding mode) and retuned by sglang PR
// #18271 (Benchmarking and Profiling: wider V-column tiles make the same
// kernel faster because each program then moves whole cache lines).  The
// Triton kernels on those pages are prior art; this is a different design
// built for 64-wide wavefronts.
//
// This file holds the column-tile kernel (KV layout), the value-row kernels
// (VK layout) and the standalone gating kernel of the unfused pair, with the
// launch dispatcher.  The row-split kernels are in gdn_rows.hip, the chunked
// kernel in gdn_chunk.hip.
//
// Work decomposition of the column tiles
//   * A workgroup serves one (sequence, k-head) -- or a slice of its G v-heads
//     when G*V/BV exceeds the wavefronts per workgroup -- so the normalised
//     q/k of that k-head are computed once and shared through LDS by all the
//     v-heads of its GQA group.
//   * Each wavefront owns one (v-head, BV-column tile): the K x BV slice of
//     the fp32 state lives in VGPRs for the whole token loop.
//   * Lane l holds columns 4*(l % LPR) .. +3 of the tile (LPR = BV/4 lanes
//     span one 16*LPR-byte row segment) and rows r = l/LPR + RG*i,
//     i = 0..RPL-1 (RG = 64/LPR row groups, RPL = K/RG rows per lane).  One
//     128-bit load per row per lane: an instruction covers RG consecutive rows
//     x BV columns, i.e. whole 128-byte lines for BV >= 32.
//   * S^T k and S^T q are reduced in-lane over the RPL rows, then across the RG
//     row groups with DPP row rotations and the gfx950 permlane16/32 swaps,
//     which leave every lane of a column with a bitwise identical sum.
//   * The output uses o = S_new^T q = gamma*(S_old^T q) + u*(k.q), so both
//     reductions run on the same state in one pass and one butterfly.
//
// The single-token kernel (CHUNK = 1) issues the state loads first and does
// the q/k normalisation and gating while they are in flight.  The multi-token
// kernel stages CHUNK tokens of normalised q/k (shared) and of v (per wave)
// in LDS, computes the gates of the chunk one token per lane, and then runs
// the dependent token loop with the state resident in VGPRs.

#include "gdn_tile.h"

namespace gdn {
namespace {

// ------------------------------------------------------- column-tile kernel
template <int K, int BV, int ACT, int CHUNK>
__global__ void __launch_bounds__(kMaxThreads)
gdn_fused_update(const FusedParams p) {
    constexpr int LPR = BV / 4;        // lanes per row segment
    constexpr int RG = kWave / LPR;    // row groups per wave
    constexpr int RPL = K / RG;        // rows per lane
    static_assert(BV % 4 == 0 && LPR >= 2 && LPR <= 16, "BV must be 8, 16, 32 or 64");
    static_assert(RPL >= 1 && K % RG == 0, "K too small for this BV");
    static_assert(CHUNK >= 1 && CHUNK <= kWave, "one gate lane per staged token");

    extern __shared__ __align__(16) float lds[];
    float* qs = lds;                        // [CHUNK][K] normalised, permuted q
    float* ks = lds + CHUNK * K;            // [CHUNK][K] normalised, permuted k

    const int waves = blockDim.x / kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;

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

    const int nvb = p.V / BV;
    const int unit = gslice * waves + wave;    // (v-head in group, tile) of this wave
    const int h = j * p.G + unit / nvb;
    const int col = (unit % nvb) * BV + 4 * (lane % LPR);
    const int rg = lane / LPR;

    const size_t tile_elems = static_cast<size_t>(K) * p.V;
    // element (rg + RG*i, col) of a tile: lane offset + i row-group steps
    const uint32_t row_step = static_cast<uint32_t>(RG * p.V);
    const uint32_t lane_elem = static_cast<uint32_t>(rg * p.V + col);
    const TileIO tio = tile_io(p.pool, p.state_bf16, static_cast<size_t>(slot) * p.Hv + h,
                               tile_elems, lane_elem);

    // State tile -> VGPRs.  Issued first so the loads overlap the staging of
    // the first chunk; unpacked after its barrier.
    const auto rows_at = [=](int i) { return i * row_step; };
    u32x4 raw[RPL];
    tile_issue<RPL>(tio, rows_at, raw);
    float4 S[RPL];

    // ---- staging of one chunk: normalised q/k (shared by the workgroup),
    // permuted so that a lane's rows rg + RG*i sit at rg*RPL + i, then the
    // gates and v of this wave's head (CHUNK > 1: lane tau holds token tau's
    // gates, v rows go to LDS)
    float gam, bet;
    float4 vdirect;
    float* vs = lds + 2 * CHUNK * K + wave * (CHUNK * BV);   // [CHUNK][BV] (CHUNK > 1)
    const int tcol = col - (unit % nvb) * BV;                 // column within the tile
    const auto stage = [&](int64_t c0, int nt) {
        stage_qk<K, ACT>(p, qs, ks, j, c0, nt, wave, waves, lane,
                         [](int kappa) { return (kappa % RG) * RPL + kappa / RG; });
        gam = 1.0f;
        bet = 0.0f;
        vdirect = make_float4(0.f, 0.f, 0.f, 0.f);
        if constexpr (CHUNK == 1) {
            token_gates<ACT>(p, c0, h, gam, bet);
            float vv[4];
            load_act<ACT, 4>(p.v, c0 * p.v_stride + static_cast<int64_t>(h) * p.V + col, vv);
            vdirect = make_float4(vv[0], vv[1], vv[2], vv[3]);
        } else {
            if (lane < nt) token_gates<ACT>(p, c0 + lane, h, gam, bet);
            // RG tokens per pass, LPR lanes per token
            for (int tok = rg; tok < nt; tok += RG) {
                float vv[4];
                load_act<ACT, 4>(p.v, (c0 + tok) * p.v_stride + static_cast<int64_t>(h) * p.V + col, vv);
                *reinterpret_cast<float4*>(vs + tok * BV + tcol) = make_float4(vv[0], vv[1], vv[2], vv[3]);
            }
        }
        lds_barrier();
    };

    // The loop is rotated so the first chunk is staged while the state loads
    // are in flight, and the raw state words die at the unpack.
    int64_t c0 = t0;
    int nt = static_cast<int>(t1 - c0 < CHUNK ? t1 - c0 : CHUNK);
    stage(c0, nt);
    tile_unpack<RPL>(tio.bf16, raw, S);
    for (;;) {
        // ---- the dependent token loop
        for (int tau = 0; tau < nt; ++tau) {
            const int64_t t = c0 + tau;
            float gamma, beta;
            float4 vv;
            if constexpr (CHUNK == 1) {
                gamma = gam;
                beta = bet;
                vv = vdirect;
            } else {
                gamma = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gam), tau));
                beta = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bet), tau));
                vv = *reinterpret_cast<const float4*>(vs + tau * BV + tcol);
            }
            float kh[RPL], qh[RPL];
            lds_read<RPL>(ks + tau * K + rg * RPL, kh);
            lds_read<RPL>(qs + tau * K + rg * RPL, qh);

            // partial S^T k, S^T q and k.q over this lane's rows
            float pk0 = 0.f, pk1 = 0.f, pk2 = 0.f, pk3 = 0.f;
            float pq0 = 0.f, pq1 = 0.f, pq2 = 0.f, pq3 = 0.f, kq = 0.f;
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                pk0 = __builtin_fmaf(S[i].x, kh[i], pk0);
                pk1 = __builtin_fmaf(S[i].y, kh[i], pk1);
                pk2 = __builtin_fmaf(S[i].z, kh[i], pk2);
                pk3 = __builtin_fmaf(S[i].w, kh[i], pk3);
                pq0 = __builtin_fmaf(S[i].x, qh[i], pq0);
                pq1 = __builtin_fmaf(S[i].y, qh[i], pq1);
                pq2 = __builtin_fmaf(S[i].z, qh[i], pq2);
                pq3 = __builtin_fmaf(S[i].w, qh[i], pq3);
                kq = __builtin_fmaf(kh[i], qh[i], kq);
            }
            pk0 = sum_row_groups<LPR>(pk0);
            pk1 = sum_row_groups<LPR>(pk1);
            pk2 = sum_row_groups<LPR>(pk2);
            pk3 = sum_row_groups<LPR>(pk3);
            pq0 = sum_row_groups<LPR>(pq0);
            pq1 = sum_row_groups<LPR>(pq1);
            pq2 = sum_row_groups<LPR>(pq2);
            pq3 = sum_row_groups<LPR>(pq3);
            kq = sum_row_groups<LPR>(kq);

            // delta and output: r = gamma*S_old^T k, u = beta*(v - r),
            // o = gamma*S_old^T q + u*(k.q)
            float4 u, o;
            u.x = beta * (vv.x - gamma * pk0);
            u.y = beta * (vv.y - gamma * pk1);
            u.z = beta * (vv.z - gamma * pk2);
            u.w = beta * (vv.w - gamma * pk3);
            o.x = __builtin_fmaf(u.x, kq, gamma * pq0);
            o.y = __builtin_fmaf(u.y, kq, gamma * pq1);
            o.z = __builtin_fmaf(u.z, kq, gamma * pq2);
            o.w = __builtin_fmaf(u.w, kq, gamma * pq3);
            if (rg == 0)
                store4_act<ACT>(p.out, (t * p.Hv + h) * static_cast<int64_t>(p.V) + col, o);

            // decay + rank-1 update
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                S[i].x = __builtin_fmaf(kh[i], u.x, gamma * S[i].x);
                S[i].y = __builtin_fmaf(kh[i], u.y, gamma * S[i].y);
                S[i].z = __builtin_fmaf(kh[i], u.z, gamma * S[i].z);
                S[i].w = __builtin_fmaf(kh[i], u.w, gamma * S[i].w);
            }
            if (p.inter) {
                const TileIO it = tile_io(p.inter, p.state_bf16, static_cast<size_t>(t) * p.Hv + h,
                                          tile_elems, lane_elem);
                const uint32_t rs = opaque_uniform(row_step);
                tile_store_all<RPL>(it, [=](int i) { return i * rs; }, S);
            }
        }
        c0 += CHUNK;
        if (c0 >= t1) break;
        nt = static_cast<int>(t1 - c0 < CHUNK ? t1 - c0 : CHUNK);
        lds_barrier();   // the next chunk reuses the LDS
        stage(c0, nt);
    }

    if (p.write_final) tile_store_all<RPL>(tio, rows_at, S);
}


// -------------------------------------------------------- value-row kernels
// State stored transposed ("VK": each of the V value-rows holds its K key
// entries contiguously).  A wavefront owns whole value-rows.  LPR = K/8 lanes
// span one row and each lane holds keys 4c..4c+3 and 4(c+LPR)..+3
// (c = lane % LPR), so a 128-bit instruction moves RG = 64/LPR rows, two
// half-rows of 256 bytes per row at K = 128.  Lane l holds rows
// vw*RPW + RG*i + l/LPR (i < RPL).  Every reduction over K -- the q/k norms,
// S^T k, S^T q and k.q -- stays inside the wavefront (LPR-lane DPP/permlane
// sums), and the update of value-row i needs only that row's u_i, so rows are
// processed one after another.  The single-token kernel uses no LDS and no
// barrier: its wavefronts never wait for each other.
template <int K, int V>
struct ValueRows {
    static constexpr int CPL = 2;                                   // 128-bit chunks per lane per row
    static constexpr int LPR = K / (4 * CPL);                       // lanes per row
    static constexpr int RG = kWave / LPR;                          // rows per instruction
    static constexpr int RPL = (V / RG < 8) ? V / RG : 8;           // rows per lane
    static constexpr int RPW = RPL * RG;                            // rows per wave
    static constexpr int VW = V / RPW;                              // waves per head
    static constexpr uint32_t ROW_STEP = RG * K;                    // elements between a lane's rows
    static constexpr uint32_t HALF = LPR * 4;                       // elements between a lane's chunks
};

// Loads this lane's keys of one q or k vector: chunks at 4c and 4(c+LPR).
template <int K, int ACT, int LPR>
__device__ __forceinline__ void load_keys(const void* base, int64_t row, int c, float (&x)[8]) {
    float lo[4], hi[4];
    load_act<ACT, 4>(base, row + 4 * c, lo);
    load_act<ACT, 4>(base, row + 4 * (c + LPR), hi);
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[e] = lo[e]; x[4 + e] = hi[e]; }
}

// Normalises this lane's keys of q and k (sum of squares over the LPR lanes of
// a row, one rsqrt each; q carries the query scale) and forms k.q.  Both
// value-row kernels call it, so their norms round identically.
template <int LPR>
__device__ __forceinline__ void normalize_keys(const float (&qx)[8], const float (&kx)[8], float scale,
                                               float eps, float (&qh)[8], float (&kh)[8], float& kq) {
    float ssq = 0.f, ssk = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        ssq = __builtin_fmaf(qx[e], qx[e], ssq);
        ssk = __builtin_fmaf(kx[e], kx[e], ssk);
    }
    ssq = sum_lane_groups<LPR>(ssq);
    ssk = sum_lane_groups<LPR>(ssk);
    const float fq = scale * rsqrtf(ssq + eps);
    const float fk = rsqrtf(ssk + eps);
    kq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        qh[e] = qx[e] * fq;
        kh[e] = kx[e] * fk;
        kq = __builtin_fmaf(kh[e], qh[e], kq);
    }
    kq = sum_lane_groups<LPR>(kq);
}

// One value-row step: S^T k and S^T q of row i (this lane's keys, then the
// LPR-lane sum), u = beta*(v - gamma*S^T k), o = gamma*S^T q + u*(k.q), and
// the decayed rank-1 update of the row.  Returns o.
template <int LPR>
__device__ __forceinline__ float value_row_step(float4 (&Si)[2], const float (&kh)[8],
                                                const float (&qh)[8], float v, float gamma,
                                                float beta, float kq) {
    const float s8[8] = {Si[0].x, Si[0].y, Si[0].z, Si[0].w, Si[1].x, Si[1].y, Si[1].z, Si[1].w};
    float pk = s8[0] * kh[0], pq = s8[0] * qh[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) {
        pk = __builtin_fmaf(s8[e], kh[e], pk);
        pq = __builtin_fmaf(s8[e], qh[e], pq);
    }
    pk = sum_lane_groups<LPR>(pk);
    pq = sum_lane_groups<LPR>(pq);
    const float u = beta * (v - gamma * pk);
    const float o = __builtin_fmaf(u, kq, gamma * pq);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        Si[hh].x = __builtin_fmaf(kh[4 * hh + 0], u, gamma * Si[hh].x);
        Si[hh].y = __builtin_fmaf(kh[4 * hh + 1], u, gamma * Si[hh].y);
        Si[hh].z = __builtin_fmaf(kh[4 * hh + 2], u, gamma * Si[hh].z);
        Si[hh].w = __builtin_fmaf(kh[4 * hh + 3], u, gamma * Si[hh].w);
    }
    return o;
}

// Workgroup -> (sequence, k-head, slice of wavefront units); a unit is
// (v-head of the GQA group, block of RPW value-rows).
struct VkPlace {
    int seq, j, h, vw;
};

template <int VW>
__device__ __forceinline__ VkPlace vk_place(const FusedParams& p, int wave, int waves) {
    int64_t blk = blockIdx.x;
    const int gslice = static_cast<int>(blk % p.groups_per_khead);
    blk /= p.groups_per_khead;
    VkPlace pl;
    pl.j = static_cast<int>(blk % p.Hk);
    pl.seq = static_cast<int>(blk / p.Hk);
    const int unit = gslice * waves + wave;
    pl.h = pl.j * p.G + unit / VW;
    pl.vw = unit % VW;
    return pl;
}

template <int K, int V, int ACT>
__global__ void __launch_bounds__(kMaxThreads)
gdn_vk_decode(const FusedParams p) {
    using L = ValueRows<K, V>;
    constexpr int LPR = L::LPR, RG = L::RG, RPL = L::RPL, RPW = L::RPW, VW = L::VW;
    static_assert(LPR >= 4 && RPL >= 1 && V % RPW == 0, "unsupported K/V pair");

    const int waves = blockDim.x / kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const VkPlace pl = vk_place<VW>(p, wave, waves);
    const int32_t slot = p.state_idx[pl.seq];
    if (slot < 0) return;  // padded: touch nothing
    const int64_t t = pl.seq;
    const int h = pl.h;
    const int c = lane % LPR;
    const int row0 = pl.vw * RPW + lane / LPR;   // this lane's rows: row0 + RG*i

    // small loads first; they return while the state streams in
    float qx[8], kx[8];
    load_keys<K, ACT, LPR>(p.q, t * p.q_stride + static_cast<int64_t>(pl.j) * K, c, qx);
    load_keys<K, ACT, LPR>(p.k, t * p.k_stride + static_cast<int64_t>(pl.j) * K, c, kx);
    float gamma, beta;
    token_gates<ACT>(p, t, h, gamma, beta);
    float vv[RPL];
    const int64_t vbase = t * p.v_stride + static_cast<int64_t>(h) * V + row0;
#pragma unroll
    for (int i = 0; i < RPL; ++i) vv[i] = load_scalar<ACT>(p.v, vbase + RG * i);

    const uint32_t lane_elem = static_cast<uint32_t>(row0 * K + 4 * c);
    const TileIO tio = tile_io(p.pool, p.state_bf16, static_cast<size_t>(slot) * p.Hv + h, K * V, lane_elem);
    // group 2i+hh: chunk hh of row i
    const auto groups_at = [](int e) { return (e >> 1) * L::ROW_STEP + (e & 1) * L::HALF; };
    u32x4 raw[2 * RPL];
    tile_issue<2 * RPL>(tio, groups_at, raw);

    float qh[8], kh[8], kq;
    normalize_keys<LPR>(qx, kx, p.scale, p.eps, qh, kh, kq);
    float4 S[RPL][2];
    tile_unpack<2 * RPL>(tio.bf16, raw, reinterpret_cast<float4(&)[2 * RPL]>(S));

    const int64_t obase = (t * p.Hv + h) * static_cast<int64_t>(V) + row0;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        const float o = value_row_step<LPR>(S[i], kh, qh, vv[i], gamma, beta, kq);
        if (c == 0) store1_act<ACT>(p.out, obase + RG * i, o);
    }
    if (p.inter) {
        const TileIO it = tile_io(p.inter, p.state_bf16, static_cast<size_t>(t) * p.Hv + h, K * V, lane_elem);
        tile_store_all<2 * RPL>(it, groups_at, reinterpret_cast<const float4(&)[2 * RPL]>(S));
    }
    if (p.write_final)
        tile_store_all<2 * RPL>(tio, groups_at, reinterpret_cast<const float4(&)[2 * RPL]>(S));
}

// Raw (widened) q and k of tokens [c0, c0+nt) into qs/ks ([nt][K] each),
// spread over all lanes of the workgroup.
template <int K, int ACT>
__device__ __forceinline__ void stage_raw_qk(const FusedParams& p, float* qs, float* ks, int j,
                                             int64_t c0, int nt, int tid, int threads) {
    for (int e = tid * 4; e < 2 * nt * K; e += threads * 4) {
        const int vec = e / K, kk = e % K;
        const int tok = vec >> 1;
        const bool is_k = vec & 1;
        float x[4];
        load_act<ACT, 4>(is_k ? p.k : p.q,
                         (c0 + tok) * (is_k ? p.k_stride : p.q_stride) + static_cast<int64_t>(j) * K + kk, x);
        *reinterpret_cast<float4*>((is_k ? ks : qs) + tok * K + kk) = make_float4(x[0], x[1], x[2], x[3]);
    }
}

// Multi-token value-row kernel: the token loop keeps the state in VGPRs;
// chunks of CHUNK tokens of raw q/k (shared by the workgroup, one barrier per
// chunk), of v (per wave) and of the gates (one token per lane) are staged in
// LDS, and each wavefront normalises q/k itself exactly as the single-token
// kernel does.
template <int K, int V, int ACT, int CHUNK>
__global__ void __launch_bounds__(kMaxThreads)
gdn_vk_multi(const FusedParams p) {
    using L = ValueRows<K, V>;
    constexpr int LPR = L::LPR, RG = L::RG, RPL = L::RPL, RPW = L::RPW, VW = L::VW;
    static_assert(LPR >= 4 && RPL >= 1 && V % RPW == 0, "unsupported K/V pair");

    extern __shared__ __align__(16) float lds[];
    float* qs = lds;                 // [CHUNK][K] raw q
    float* ks = lds + CHUNK * K;     // [CHUNK][K] raw k

    const int waves = blockDim.x / kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const VkPlace pl = vk_place<VW>(p, wave, waves);
    const int32_t slot = p.state_idx[pl.seq];
    int64_t t0, t1;
    if (p.cu_seqlens) {
        t0 = p.cu_seqlens[pl.seq];
        t1 = p.cu_seqlens[pl.seq + 1];
    } else {
        t0 = static_cast<int64_t>(pl.seq) * p.T;
        t1 = t0 + p.T;
    }
    if (slot < 0 || t1 <= t0) return;  // padded or empty: touch nothing
    const int h = pl.h;
    const int c = lane % LPR;
    const int rg = lane / LPR;
    const int row0 = pl.vw * RPW + rg;
    float* vs = lds + 2 * CHUNK * K + wave * (CHUNK * RPW);   // [CHUNK][RPW] this wave's v

    const uint32_t lane_elem = static_cast<uint32_t>(row0 * K + 4 * c);
    const TileIO tio = tile_io(p.pool, p.state_bf16, static_cast<size_t>(slot) * p.Hv + h, K * V, lane_elem);
    const auto groups_at = [](int e) { return (e >> 1) * L::ROW_STEP + (e & 1) * L::HALF; };
    u32x4 raw[2 * RPL];
    tile_issue<2 * RPL>(tio, groups_at, raw);
    float4 S[RPL][2];
    float4 (&Sf)[2 * RPL] = reinterpret_cast<float4(&)[2 * RPL]>(S);

    // staging of one chunk: raw q/k (shared), the gates (lane tau holds token
    // tau's) and v of this wave's rows, permuted so lane (rg, i) reads
    // rg*RPL + i
    float gam, bet;
    const auto stage = [&](int64_t c0, int nt) {
        stage_raw_qk<K, ACT>(p, qs, ks, pl.j, c0, nt, threadIdx.x, blockDim.x);
        gam = 1.0f;
        bet = 0.0f;
        if (lane < nt) token_gates<ACT>(p, c0 + lane, h, gam, bet);
        for (int e = lane; e < nt * RPW; e += kWave) {
            const int tok = e / RPW, r = e % RPW;
            vs[tok * RPW + (r % RG) * RPL + r / RG] =
                load_scalar<ACT>(p.v, (c0 + tok) * p.v_stride + static_cast<int64_t>(h) * V +
                                          pl.vw * RPW + r);
        }
        lds_barrier();
    };

    // Rotated loop: the first chunk is staged while the state loads are in
    // flight, and the raw state words die at the unpack.
    int64_t c0 = t0;
    int nt = static_cast<int>(t1 - c0 < CHUNK ? t1 - c0 : CHUNK);
    stage(c0, nt);
    tile_unpack<2 * RPL>(tio.bf16, raw, Sf);
    for (;;) {
        for (int tau = 0; tau < nt; ++tau) {
            const int64_t t = c0 + tau;
            const float gamma = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gam), tau));
            const float beta = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bet), tau));
            float kx[8], qx[8], vv[RPL];
            lds_read<4>(ks + tau * K + 4 * c, reinterpret_cast<float(&)[4]>(kx[0]));
            lds_read<4>(ks + tau * K + 4 * (c + LPR), reinterpret_cast<float(&)[4]>(kx[4]));
            lds_read<4>(qs + tau * K + 4 * c, reinterpret_cast<float(&)[4]>(qx[0]));
            lds_read<4>(qs + tau * K + 4 * (c + LPR), reinterpret_cast<float(&)[4]>(qx[4]));
            lds_read<RPL>(vs + tau * RPW + rg * RPL, vv);
            float kh[8], qh[8], kq;
            normalize_keys<LPR>(qx, kx, p.scale, p.eps, qh, kh, kq);

            const int64_t obase = (t * p.Hv + h) * static_cast<int64_t>(V) + row0;
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                const float o = value_row_step<LPR>(S[i], kh, qh, vv[i], gamma, beta, kq);
                if (c == 0) store1_act<ACT>(p.out, obase + RG * i, o);
            }
            if (p.inter) {
                const TileIO it =
                    tile_io(p.inter, p.state_bf16, static_cast<size_t>(t) * p.Hv + h, K * V, lane_elem);
                tile_store_all<2 * RPL>(it, groups_at, Sf);
            }
        }
        c0 += CHUNK;
        if (c0 >= t1) break;
        nt = static_cast<int>(t1 - c0 < CHUNK ? t1 - c0 : CHUNK);
        lds_barrier();   // the next chunk reuses the LDS
        stage(c0, nt);
    }

    if (p.write_final) tile_store_all<2 * RPL>(tio, groups_at, Sf);
}


// ---------------------------------------------------------- gating kernel
// The standalone gating step of the unfused pair (vLLM PR #35777,
// implementation section: the gating kernel that the fused op absorbs):
// g = -exp(A_log)*softplus(a + dt_bias) and beta = sigmoid(b), written as
// fp32 [N, H_v].  One thread per (token, v-head).
template <int ACT>
__global__ void __launch_bounds__(256)
gdn_gating_kernel(const void* a, const void* b, const float* A_log, const float* dt_bias,
                  float* g, float* beta, int64_t n, int Hv, int G, int64_t ab_stride,
                  int32_t ab_khead) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (e >= n) return;
    const int64_t t = e / Hv;
    const int h = static_cast<int>(e % Hv);
    const int64_t src = t * ab_stride + static_cast<int64_t>(h / G) * ab_khead + h % G;
    float gv, bv;
    gate_values(load_scalar<ACT>(a, src), load_scalar<ACT>(b, src), A_log[h], dt_bias[h], gv, bv);
    g[e] = gv;
    beta[e] = bv;
}

// ------------------------------------------------------------ instance table

// A (K, BV) pair has an instance when the K x BV fp32 tile fits in at most
// 128 VGPRs per lane.
constexpr bool valid_pair(int K, int BV) { return K * BV <= 128 * kWave; }

template <int K, int BV, int ACT, int CHUNK>
KernelFn pick() {
    if constexpr (valid_pair(K, BV)) return &gdn_fused_update<K, BV, ACT, CHUNK>;
    else return nullptr;
}

template <int K, int ACT, int CHUNK>
KernelFn by_bv(int BV) {
    switch (BV) {
        case 8: return pick<K, 8, ACT, CHUNK>();
        case 16: return pick<K, 16, ACT, CHUNK>();
        case 32: return pick<K, 32, ACT, CHUNK>();
        case 64: return pick<K, 64, ACT, CHUNK>();
        default: return nullptr;
    }
}

template <int ACT, int CHUNK>
KernelFn by_k(int K, int BV) {
    switch (K) {
        case 32: return by_bv<32, ACT, CHUNK>(BV);
        case 64: return by_bv<64, ACT, CHUNK>(BV);
        case 128: return by_bv<128, ACT, CHUNK>(BV);
        case 256: return by_bv<256, ACT, CHUNK>(BV);
        default: return nullptr;
    }
}

KernelFn select_columns(int K, int BV, int act, int multi_token) {
    if (act == 0) return multi_token ? by_k<0, kChunkTokens>(K, BV) : by_k<0, 1>(K, BV);
    return multi_token ? by_k<1, kChunkTokens>(K, BV) : by_k<1, 1>(K, BV);
}
template <int K, int V, int ACT>
KernelFn pick_vk(int multi) {
    return multi ? &gdn_vk_multi<K, V, ACT, kChunkTokens> : &gdn_vk_decode<K, V, ACT>;
}

template <int K, int ACT>
KernelFn vk_by_v(int V, int multi) {
    switch (V) {
        case 32: return pick_vk<K, 32, ACT>(multi);
        case 64: return pick_vk<K, 64, ACT>(multi);
        case 128: return pick_vk<K, 128, ACT>(multi);
        case 256: return pick_vk<K, 256, ACT>(multi);
        default: return nullptr;
    }
}

KernelFn select_vk(int K, int V, int act, int multi) {
    switch (K) {
        case 32: return act ? vk_by_v<32, 1>(V, multi) : vk_by_v<32, 0>(V, multi);
        case 64: return act ? vk_by_v<64, 1>(V, multi) : vk_by_v<64, 0>(V, multi);
        case 128: return act ? vk_by_v<128, 1>(V, multi) : vk_by_v<128, 0>(V, multi);
        case 256: return act ? vk_by_v<256, 1>(V, multi) : vk_by_v<256, 0>(V, multi);
        default: return nullptr;
    }
}

template <int K, int V>
int vk_rows_of() { return ValueRows<K, V>::RPW; }

template <int K>
int vk_rows_by_v(int V) {
    switch (V) {
        case 32: return vk_rows_of<K, 32>();
        case 64: return vk_rows_of<K, 64>();
        case 128: return vk_rows_of<K, 128>();
        case 256: return vk_rows_of<K, 256>();
        default: return 0;
    }
}

}  // namespace

int vk_rows_per_wave(int K, int V) {
    if (!select_vk(K, V, 0, 0)) return 0;
    switch (K) {
        case 32: return vk_rows_by_v<32>(V);
        case 64: return vk_rows_by_v<64>(V);
        case 128: return vk_rows_by_v<128>(V);
        case 256: return vk_rows_by_v<256>(V);
        default: return 0;
    }
}

bool instance_exists(int K, int block_v) {
    return select_columns(K, block_v, 0, 0) != nullptr;
}

int lds_bytes_for(const LaunchShape& s, int V) {
    int floats = 2 * s.chunk * s.K;                          // normalised q and k
    if (s.kind == kKindColumns && s.multi_token)
        floats += s.waves * s.chunk * s.block_v;             // per-wave v rows
    if (s.kind == kKindRows) {
        const int heads = s.waves / (s.K / s.block_k);
        if (s.multi_token)  // staged v rows per head, partial sums double-buffered
            floats += heads * s.chunk * V + 2 * s.waves * (2 * V + 4);
        else
            floats += s.waves * (2 * V + 4);                  // per-wave partial sums
    }
    if (s.kind == kKindValueRows)                             // single token: no LDS at all
        floats = s.multi_token ? 2 * s.chunk * s.K + s.waves * s.chunk * s.block_v : 0;
    return floats * static_cast<int>(sizeof(float));
}

hipError_t launch_gating(const void* a, const void* b, const float* A_log, const float* dt_bias,
                         float* g, float* beta, int64_t n, int Hv, int G, int64_t ab_stride,
                         int32_t ab_khead, int act, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
    void* fn = act ? reinterpret_cast<void*>(&gdn_gating_kernel<1>)
                   : reinterpret_cast<void*>(&gdn_gating_kernel<0>);
    void* args[] = {const_cast<void**>(&a), const_cast<void**>(&b), const_cast<float**>(&A_log),
                    const_cast<float**>(&dt_bias), &g, &beta, &n, &Hv, &G, &ab_stride, &ab_khead};
    return hipLaunchKernel(fn, dim3(blocks), dim3(256), args, 0, stream);
}

hipError_t launch_fused(const LaunchShape& s, const FusedParams& p, hipStream_t stream) {
    KernelFn fn = s.kind == kKindRows        ? select_rows(s.K, p.V, s.act, s.rows_rpl_max, s.multi_token)
                  : s.kind == kKindValueRows ? select_vk(s.K, p.V, s.act, s.multi_token)
                                             : select_columns(s.K, s.block_v, s.act, s.multi_token);
    if (!fn) return hipErrorInvalidDeviceFunction;
    void* args[] = {const_cast<FusedParams*>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(static_cast<unsigned>(s.groups)),
                           dim3(s.waves * kWave), args, static_cast<size_t>(s.lds_bytes), stream);
}

}  // namespace gdn
