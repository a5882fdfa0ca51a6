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
// Work decomposition
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

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kWave = 64;
constexpr int kMaxThreads = 512;

// The state streams through HBM once per call (read, then written back), so
// its loads and stores carry the non-temporal hint.  They are raw buffer
// operations on a resource that spans exactly one K x V tile: the tile base
// sits in SGPRs, each lane keeps one 32-bit byte offset in a VGPR, and the
// row-group step is a scalar offset -- no 64-bit address per row stays live
// between the loads and the final stores.  Offsets past the tile would be
// clamped by the hardware (loads return 0, stores are dropped).
constexpr int kBufNonTemporal = 2;           // cache-policy bit "nt" (gfx94x/gfx950)
// Word 3 of a gfx9-family raw buffer resource: 32-bit data format, no swizzle.
constexpr int kBufWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const float* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, static_cast<int>(bytes),
                                             kBufWord3);
}

__device__ __forceinline__ float4 load_state(__amdgpu_buffer_rsrc_t r, uint32_t lane_bytes,
                                             uint32_t row_bytes) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, lane_bytes, row_bytes, kBufNonTemporal);
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                       __uint_as_float(v[3]));
}

__device__ __forceinline__ void store_state(__amdgpu_buffer_rsrc_t r, uint32_t lane_bytes,
                                            uint32_t row_bytes, const float4& s) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = {__float_as_uint(s.x), __float_as_uint(s.y), __float_as_uint(s.z),
                     __float_as_uint(s.w)};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, lane_bytes, row_bytes, kBufNonTemporal);
}

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// N consecutive activation elements starting at element `e`, widened to fp32.
// ACT 0 = fp32, 1 = bf16.  The start is aligned to min(16, N*size) bytes.
template <int ACT, int N>
__device__ __forceinline__ void load_act(const void* base, int64_t e, float (&x)[N]) {
    if constexpr (ACT == 0) {
        const float* p = static_cast<const float*>(base) + e;
        if constexpr (N % 4 == 0) {
#pragma unroll
            for (int i = 0; i < N / 4; ++i) {
                const float4 t = reinterpret_cast<const float4*>(p)[i];
                x[4 * i + 0] = t.x; x[4 * i + 1] = t.y; x[4 * i + 2] = t.z; x[4 * i + 3] = t.w;
            }
        } else if constexpr (N == 2) {
            const float2 t = *reinterpret_cast<const float2*>(p);
            x[0] = t.x; x[1] = t.y;
        } else {
#pragma unroll
            for (int i = 0; i < N; ++i) x[i] = p[i];
        }
    } else {
        const uint16_t* p = static_cast<const uint16_t*>(base) + e;
        if constexpr (N % 8 == 0) {
#pragma unroll
            for (int i = 0; i < N / 8; ++i) {
                const uint4 t = reinterpret_cast<const uint4*>(p)[i];
                const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[8 * i + 2 * j] = bf16_lo(w[j]);
                    x[8 * i + 2 * j + 1] = bf16_hi(w[j]);
                }
            }
        } else if constexpr (N == 4) {
            const uint2 t = *reinterpret_cast<const uint2*>(p);
            x[0] = bf16_lo(t.x); x[1] = bf16_hi(t.x); x[2] = bf16_lo(t.y); x[3] = bf16_hi(t.y);
        } else if constexpr (N == 2) {
            const uint32_t t = *reinterpret_cast<const uint32_t*>(p);
            x[0] = bf16_lo(t); x[1] = bf16_hi(t);
        } else {
#pragma unroll
            for (int i = 0; i < N; ++i) x[i] = __uint_as_float(uint32_t(p[i]) << 16);
        }
    }
}

template <int ACT>
__device__ __forceinline__ float load_scalar(const void* base, int64_t e) {
    if constexpr (ACT == 0) return static_cast<const float*>(base)[e];
    else return __uint_as_float(uint32_t(static_cast<const uint16_t*>(base)[e]) << 16);
}

// Four consecutive output elements (16-byte aligned for fp32, 8 for bf16).
template <int ACT>
__device__ __forceinline__ void store4_act(void* base, int64_t e, float4 o) {
    if constexpr (ACT == 0) {
        *reinterpret_cast<float4*>(static_cast<float*>(base) + e) = o;
    } else {
        uint2 w;
        w.x = bf16_rne(o.x) | (bf16_rne(o.y) << 16);
        w.y = bf16_rne(o.z) | (bf16_rne(o.w) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + e) = w;
    }
}

// ------------------------------------------------------------ cross-lane sums
// Rotation by CTRL within 16-lane DPP rows (0x120 + n = row_ror:n).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// x + x[lane ^ 16]: odd 16-lane rows swap with even rows; the first result
// always holds the even row's value, so both rows add in the same order.
__device__ __forceinline__ float sum_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// x + x[lane ^ 32]: the upper half-wave swaps with the lower half-wave.
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over all lanes with the same (lane % LPR): the row groups of a tile.
template <int LPR>
__device__ __forceinline__ float sum_row_groups(float x) {
    static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "power-of-two row width");
    if constexpr (LPR <= 8) x += dpp_mov<0x128>(x);  // row_ror:8
    if constexpr (LPR <= 4) x += dpp_mov<0x124>(x);  // row_ror:4
    if constexpr (LPR <= 2) x += dpp_mov<0x122>(x);  // row_ror:2
    if constexpr (LPR <= 1) x += dpp_mov<0x121>(x);  // row_ror:1
    if constexpr (LPR <= 16) x = sum_xor16(x);
    if constexpr (LPR <= 32) x = sum_xor32(x);
    return x;
}

// Sum over the 16 lanes of a DPP row.
__device__ __forceinline__ float sum_dpp_row(float x) {
    x += dpp_mov<0x128>(x);
    x += dpp_mov<0x124>(x);
    x += dpp_mov<0x122>(x);
    x += dpp_mov<0x121>(x);
    return x;
}

// Workgroup barrier that orders LDS only: global loads already in flight (the
// state tile) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ----------------------------------------------------------------- the gates
// gamma = exp(-exp(A_log) * softplus(a + dt_bias)), beta = sigmoid(b).
// softplus returns x itself above 20, where log1p(exp(x)) - x < 2.1e-9.
__device__ __forceinline__ void gates(float a, float b, float A_log, float dt_bias,
                                      float& gamma, float& beta) {
    const float x = a + dt_bias;
    const float sp = x > 20.0f ? x : log1pf(expf(x));
    gamma = expf(-expf(A_log) * sp);
    beta = 1.0f / (1.0f + expf(-b));
}

// ----------------------------------------------------------- q/k staging
// Normalises q and k of tokens [c0, c0+nt) of k-head j into qs/ks ([nt][K]
// floats each), element kappa of a token going to position POS(kappa).  Each
// 16-lane DPP row of the workgroup handles one vector (the q or the k of one
// token): K/16 elements per lane, a row reduction, one rsqrt.  q carries the
// query scale.  Every vector is reduced in the same order, whichever row
// handles it.
template <int K, int ACT, typename POS>
__device__ __forceinline__ void stage_qk(const FusedParams& p, float* qs, float* ks, int j,
                                         int64_t c0, int nt, int wave, int waves, int lane,
                                         POS pos) {
    constexpr int EPL = K / 16;
    const int lr = lane % 16;
    for (int vec = wave * 4 + lane / 16; vec < 2 * nt; vec += 4 * waves) {
        const int tok = vec >> 1;
        const bool is_k = vec & 1;
        const int64_t t = c0 + tok;
        float x[EPL];
        if (is_k)
            load_act<ACT, EPL>(p.k, t * p.k_stride + static_cast<int64_t>(j) * K + lr * EPL, x);
        else
            load_act<ACT, EPL>(p.q, t * p.q_stride + static_cast<int64_t>(j) * K + lr * EPL, x);
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
        ss = sum_dpp_row(ss);
        const float f = (is_k ? 1.0f : p.scale) * rsqrtf(ss + p.eps);
        float* dst = (is_k ? ks : qs) + tok * K;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dst[pos(lr * EPL + e)] = x[e] * f;
    }
}

// Reads N consecutive LDS floats (16-byte aligned when N % 4 == 0).
template <int N>
__device__ __forceinline__ void lds_read(const float* src, float (&x)[N]) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const float4 t = reinterpret_cast<const float4*>(src)[i];
            x[4 * i] = t.x; x[4 * i + 1] = t.y; x[4 * i + 2] = t.z; x[4 * i + 3] = t.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = src[i];
    }
}

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
    const uint32_t tile_bytes = static_cast<uint32_t>(tile_elems * sizeof(float));
    const __amdgpu_buffer_rsrc_t tile_r =
        tile_rsrc(p.pool + (static_cast<size_t>(slot) * p.Hv + h) * tile_elems, tile_bytes);
    // element (rg + RG*i, col) of a tile: lane offset + i row-group steps
    const uint32_t row_step = static_cast<uint32_t>(RG * p.V * sizeof(float));
    const uint32_t lane_bytes = static_cast<uint32_t>((rg * p.V + col) * sizeof(float));

    // State tile -> VGPRs.  Issued first so the loads overlap the set-up below.
    float4 S[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i)
        S[i] = load_state(tile_r, lane_bytes, i * row_step);

    const float A_log = p.A_log[h];
    const float dt_bias = p.dt_bias[h];

    for (int64_t c0 = t0; c0 < t1; c0 += CHUNK) {
        const int nt = static_cast<int>(t1 - c0 < CHUNK ? t1 - c0 : CHUNK);

        // ---- stage: normalised q/k of the chunk (shared by the workgroup),
        // permuted so that a lane's rows rg + RG*i sit at rg*RPL + i
        stage_qk<K, ACT>(p, qs, ks, j, c0, nt, wave, waves, lane,
                         [](int kappa) { return (kappa % RG) * RPL + kappa / RG; });

        // ---- gates and v of the chunk (per wave)
        float gam = 1.0f, bet = 0.0f;   // CHUNK > 1: lane tau holds token tau's gates
        float4 vdirect = make_float4(0.f, 0.f, 0.f, 0.f);
        float* vs = lds + 2 * CHUNK * K + wave * (CHUNK * BV);   // [CHUNK][BV] (CHUNK > 1)
        if constexpr (CHUNK == 1) {
            gates(load_scalar<ACT>(p.a, c0 * p.Hv + h), load_scalar<ACT>(p.b, c0 * p.Hv + h),
                  A_log, dt_bias, gam, bet);
            float vv[4];
            load_act<ACT, 4>(p.v, c0 * p.v_stride + static_cast<int64_t>(h) * p.V + col, vv);
            vdirect = make_float4(vv[0], vv[1], vv[2], vv[3]);
        } else {
            if (lane < nt)
                gates(load_scalar<ACT>(p.a, (c0 + lane) * p.Hv + h),
                      load_scalar<ACT>(p.b, (c0 + lane) * p.Hv + h), A_log, dt_bias, gam, bet);
            // v rows of this wave's tile: RG tokens per pass, LPR lanes per token
            const int tcol = col - (unit % nvb) * BV;    // column within the tile
            for (int tok = rg; tok < nt; tok += RG) {
                float vv[4];
                load_act<ACT, 4>(p.v, (c0 + tok) * p.v_stride + static_cast<int64_t>(h) * p.V + col, vv);
                *reinterpret_cast<float4*>(vs + tok * BV + tcol) = make_float4(vv[0], vv[1], vv[2], vv[3]);
            }
        }
        lds_barrier();

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
                vv = *reinterpret_cast<const float4*>(vs + tau * BV + (col - (unit % nvb) * BV));
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
                const __amdgpu_buffer_rsrc_t it_r =
                    tile_rsrc(p.inter + (static_cast<size_t>(t) * p.Hv + h) * tile_elems, tile_bytes);
#pragma unroll
                for (int i = 0; i < RPL; ++i)
                    store_state(it_r, lane_bytes, i * row_step, S[i]);
            }
        }
        if (c0 + CHUNK < t1) lds_barrier();   // the next chunk reuses the LDS
    }

    if (p.write_final) {
#pragma unroll
        for (int i = 0; i < RPL; ++i)
            store_state(tile_r, lane_bytes, i * row_step, S[i]);
    }
}


// ----------------------------------------------------------- row-split kernel
// Single-token decode with whole rows per wavefront.  LPR = V/4 lanes cover
// one V-column row, so each 128-bit load or store instruction of a wave moves
// RG = 64/LPR consecutive rows: one contiguous kilobyte of the tile.  Lane l
// holds columns 4*(l % LPR)..+3 of rows kw*RPW + RG*i + l/LPR (i < RPL); the
// K rows of a head are split over KW wavefronts.  S^T k, S^T q and k.q are
// reduced in-lane, across the wave's row groups with permlane swaps, and
// across the KW wavefronts of the head through LDS, summed in a fixed order
// so every wave derives the same u.
template <int K, int V>
struct RowSplit {
    static constexpr int LPR = V / 4;                          // lanes per row
    static constexpr int RG = kWave / LPR;                     // rows per instruction
    static constexpr int RPL = (K / RG < 16) ? K / RG : 16;    // rows per lane
    static constexpr int RPW = RPL * RG;                       // rows per wave
    static constexpr int KW = K / RPW;                         // waves per head
    static constexpr int PART = 2 * V + 4;                     // partial sums per wave (floats)
};

template <int K, int V, int ACT>
__global__ void __launch_bounds__(kMaxThreads)
gdn_decode_rows(const FusedParams p) {
    using L = RowSplit<K, V>;
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

    constexpr uint32_t tile_bytes = static_cast<uint32_t>(K * V * sizeof(float));
    const __amdgpu_buffer_rsrc_t tile_r =
        tile_rsrc(p.pool + (static_cast<size_t>(slot) * p.Hv + h) * (K * V), tile_bytes);
    constexpr uint32_t row_step = RG * V * sizeof(float);   // one kilobyte
    const uint32_t lane_bytes = static_cast<uint32_t>(((kw * RPW + rg) * V + col) * sizeof(float));

    float4 S[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) S[i] = load_state(tile_r, lane_bytes, i * row_step);

    float gamma, beta;
    gates(load_scalar<ACT>(p.a, t * p.Hv + h), load_scalar<ACT>(p.b, t * p.Hv + h), p.A_log[h],
          p.dt_bias[h], gamma, beta);
    float vv[4];
    load_act<ACT, 4>(p.v, t * p.v_stride + static_cast<int64_t>(h) * V + col, vv);

    // rows kw*RPW + RG*i + rg of the head sit at kw*RPW + rg*RPL + i
    stage_qk<K, ACT>(p, qs, ks, j, t, 1, wave, waves, lane, [](int kappa) {
        const int r = kappa % RPW;
        return (kappa - r) + (r % RG) * RPL + r / RG;
    });
    lds_barrier();

    float kh[RPL], qh[RPL];
    lds_read<RPL>(ks + kw * RPW + rg * RPL, kh);
    lds_read<RPL>(qs + kw * RPW + rg * RPL, qh);
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

    float* mine = part + (hl * KW + kw) * L::PART;
    if (rg == 0) {
        *reinterpret_cast<float4*>(mine + col) = make_float4(pk[0], pk[1], pk[2], pk[3]);
        *reinterpret_cast<float4*>(mine + V + col) = make_float4(pq[0], pq[1], pq[2], pq[3]);
        if (lane == 0) mine[2 * V] = kq;
    }
    lds_barrier();

    float4 PK = make_float4(0.f, 0.f, 0.f, 0.f), PQ = PK;
    float KQ = 0.f;
    const float* head_part = part + hl * KW * L::PART;
#pragma unroll
    for (int w = 0; w < KW; ++w) {
        const float4 a4 = *reinterpret_cast<const float4*>(head_part + w * L::PART + col);
        const float4 b4 = *reinterpret_cast<const float4*>(head_part + w * L::PART + V + col);
        PK.x += a4.x; PK.y += a4.y; PK.z += a4.z; PK.w += a4.w;
        PQ.x += b4.x; PQ.y += b4.y; PQ.z += b4.z; PQ.w += b4.w;
        KQ += head_part[w * L::PART + 2 * V];
    }

    float4 u, o;
    u.x = beta * (vv[0] - gamma * PK.x);
    u.y = beta * (vv[1] - gamma * PK.y);
    u.z = beta * (vv[2] - gamma * PK.z);
    u.w = beta * (vv[3] - gamma * PK.w);
    o.x = __builtin_fmaf(u.x, KQ, gamma * PQ.x);
    o.y = __builtin_fmaf(u.y, KQ, gamma * PQ.y);
    o.z = __builtin_fmaf(u.z, KQ, gamma * PQ.z);
    o.w = __builtin_fmaf(u.w, KQ, gamma * PQ.w);
    if (kw == 0 && rg == 0) store4_act<ACT>(p.out, (t * p.Hv + h) * static_cast<int64_t>(V) + col, o);

#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        S[i].x = __builtin_fmaf(kh[i], u.x, gamma * S[i].x);
        S[i].y = __builtin_fmaf(kh[i], u.y, gamma * S[i].y);
        S[i].z = __builtin_fmaf(kh[i], u.z, gamma * S[i].z);
        S[i].w = __builtin_fmaf(kh[i], u.w, gamma * S[i].w);
    }
    if (p.inter) {
        const __amdgpu_buffer_rsrc_t it_r =
            tile_rsrc(p.inter + (static_cast<size_t>(t) * p.Hv + h) * (K * V), tile_bytes);
#pragma unroll
        for (int i = 0; i < RPL; ++i) store_state(it_r, lane_bytes, i * row_step, S[i]);
    }
    if (p.write_final) {
#pragma unroll
        for (int i = 0; i < RPL; ++i) store_state(tile_r, lane_bytes, i * row_step, S[i]);
    }
}

// ------------------------------------------------------------ instance table
using KernelFn = void (*)(FusedParams);

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
KernelFn pick_rows() {
    if constexpr (RowSplit<K, V>::KW <= 8) return &gdn_decode_rows<K, V, ACT>;
    else return nullptr;
}

template <int K, int ACT>
KernelFn rows_by_v(int V) {
    switch (V) {
        case 32: return pick_rows<K, 32, ACT>();
        case 64: return pick_rows<K, 64, ACT>();
        case 128: return pick_rows<K, 128, ACT>();
        case 256: return pick_rows<K, 256, ACT>();
        default: return nullptr;
    }
}

template <int ACT>
KernelFn rows_by_k(int K, int V) {
    switch (K) {
        case 32: return rows_by_v<32, ACT>(V);
        case 64: return rows_by_v<64, ACT>(V);
        case 128: return rows_by_v<128, ACT>(V);
        case 256: return rows_by_v<256, ACT>(V);
        default: return nullptr;
    }
}

KernelFn select_rows(int K, int V, int act) {
    return act == 0 ? rows_by_k<0>(K, V) : rows_by_k<1>(K, V);
}

template <int K, int V>
int rows_kw_of() { return RowSplit<K, V>::KW; }

template <int K>
int rows_kw_by_v(int V) {
    switch (V) {
        case 32: return rows_kw_of<K, 32>();
        case 64: return rows_kw_of<K, 64>();
        case 128: return rows_kw_of<K, 128>();
        case 256: return rows_kw_of<K, 256>();
        default: return 0;
    }
}

}  // namespace

bool instance_exists(int K, int block_v) {
    return select_columns(K, block_v, 0, 0) != nullptr;
}

int rows_waves_per_head(int K, int V) {
    if (!select_rows(K, V, 0)) return 0;
    switch (K) {
        case 32: return rows_kw_by_v<32>(V);
        case 64: return rows_kw_by_v<64>(V);
        case 128: return rows_kw_by_v<128>(V);
        case 256: return rows_kw_by_v<256>(V);
        default: return 0;
    }
}

int lds_bytes_for(const LaunchShape& s, int V) {
    int floats = 2 * s.chunk * s.K;                          // normalised q and k
    if (s.kind == kKindColumns && s.multi_token)
        floats += s.waves * s.chunk * s.block_v;             // per-wave v rows
    if (s.kind == kKindRows) floats += s.waves * (2 * V + 4);  // per-wave partial sums
    return floats * static_cast<int>(sizeof(float));
}

hipError_t launch_fused(const LaunchShape& s, const FusedParams& p, hipStream_t stream) {
    KernelFn fn = s.kind == kKindRows ? select_rows(s.K, p.V, s.act)
                                      : select_columns(s.K, s.block_v, s.act, s.multi_token);
    if (!fn) return hipErrorInvalidDeviceFunction;
    void* args[] = {const_cast<FusedParams*>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(static_cast<unsigned>(s.groups)),
                           dim3(s.waves * kWave), args, static_cast<size_t>(s.lds_bytes), stream);
}

}  // namespace gdn
