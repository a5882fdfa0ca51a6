// Chunked forward of the gated delta rule for long sequences (the prefill
// form) on gfx950 matrix cores.  It produces the same outputs and final states
// as the token-by-token update in gdn_kernels.hip, up to rounding.
//
// The chunked form.  Take one (sequence, v-head) and one chunk of C tokens.
// S0 (K x V) is the state at the chunk start.  G_t is the prefix sum of the
// log-decays g inside the chunk.  khat_t = rk_t k_t and qhat_t = rq_t q_t are
// the normalised key and query (rq includes the query scale).  Unrolling the
// per-token update over the chunk gives
//   u_t = beta_t (v_t - e^{G_t} S0^T khat_t
//                 - sum_{s<t} e^{G_t-G_s} (khat_t.khat_s) u_s)
//   o_t = e^{G_t} S0^T qhat_t + sum_{s<=t} e^{G_t-G_s} (qhat_t.khat_s) u_s
//   S'  = e^{G_last} S0 + sum_s e^{G_last-G_s} khat_s u_s^T.
// Define L[t][s] = beta_t e^{G_t-G_s} khat_t.khat_s for s < t, and
// R = diag(beta) (V - diag(e^G) Khat S0).  Then the chunk's u are
// U = (I + L)^-1 R, and O and S' each take two more products.  This is the WY
// form of the chunked gated delta rule, with chunks of 64 tokens.  In sglang
// PR #21411 (implementation section) one Triton kernel fuses its K K^T,
// triangular solve and w/u recomputation.
//
// Design.
//   * One workgroup walks every chunk of one (sequence, v-head).  Each wave
//     owns 16 value columns, and their K x 16 slice of the state stays in MFMA
//     accumulators from the first chunk to the last.  There is no chunk index
//     table and no state round trip through HBM between chunks.
//   * Everything that depends on the state is a product in which this wave's
//     own accumulators are the B operand.  The contraction index is permuted
//     so that the 8 values of a 32-deep B operand are the 4+4 rows this lane
//     already holds in two 16-row accumulator tiles.  The matching A operand
//     is read from LDS with the same permutation (two 8-byte reads).  Waves
//     therefore exchange only the state-independent matrices (raw keys and
//     queries, (I + L)^-1, the masked query-key products), which are built
//     once per chunk in LDS.
//   * Products run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  Raw
//     bf16 keys and queries are exact operands; the norms, gates and decays
//     are applied in fp32 afterwards.  An fp32 operand (the state, R, U,
//     (I + L)^-1, fp32 inputs) is split into hi + lo bf16 parts, and three
//     products (hi*hi, hi*lo, lo*hi) keep about 16 significant bits of each
//     term.
//   * Only the 16 x 16 diagonal blocks of (I + L)^-1 are formed (forward
//     substitution on 16 lanes, fp32); U follows by block forward
//     substitution with them.
//   * Two workgroup barriers per chunk.  The per-token scalars are double
//     buffered, so the next chunk's loads do not wait for the last products.

#include "gdn_chunk_common.h"

namespace gdn {
namespace {

constexpr int kVW = 16;          // value columns per wavefront
constexpr int kNT = kVW / 16;    // 16-column MFMA tiles per wavefront

// LDS layout of one workgroup (byte offsets).  The bf16 row pitches are 2 mod
// 4 dwords: the 16 lanes that one cycle of an 8-byte operand read serves (16
// consecutive rows at one column) then fall on 16 distinct bank pairs of the
// 32-bank LDS, where a pitch of 0 mod 4 dwords would put rows m and m + 8 on
// the same banks and double the time of every such read.  Those rows are only
// 8-byte aligned, so every access to them is at most 8 bytes wide.  fp32
// activations keep a hi and a lo bf16 copy of keys and queries.
template <int K, int V, int ACT>
struct ChunkPlan {
    static constexpr int NW = V / kVW;
    static constexpr int THREADS = NW * kWave;
    static constexpr int P = ACT == 0 ? 2 : 1;     // bf16 parts per input element
    static constexpr int KT = K + 4;               // pitch of [C][K] (bf16)
    static constexpr int KC = kC + 4;              // pitch of [K][C] and [C][C] (bf16)
    static constexpr int LD = 16 + 4;              // pitch of a 16 x 16 fp32 block
    static constexpr int kScalars = 7;             // beta, e^G, e^{G_last-G}, rk, rq, G hi, G lo
    static constexpr int kt = 0;                              // P x [C][KT] raw keys
    static constexpr int qt = kt + P * kC * KT * 2;           // P x [C][KT] raw queries
    static constexpr int kc = qt + P * kC * KT * 2;           // P x [K][KC] raw keys, transposed
    static constexpr int lt = kc + P * K * KC * 2;            // 4 x [16][LD] fp32: diagonal blocks of L
    static constexpr int tb = lt + 4 * 16 * LD * 4;           // 2 x [C][KC]: D_b on, -L below the diagonal
    static constexpr int pb = tb + 2 * kC * KC * 2;           // 2 x [C][KC]: masked query-key products
    static constexpr int sc = pb + 2 * kC * KC * 2;           // 2 x kScalars x [C]
    static constexpr int bytes = sc + 2 * kScalars * kC * 4;
    static_assert(V % kVW == 0 && K % 32 == 0, "16-column waves, 32-deep key steps");
    static_assert((KT / 2) % 4 == 2 && (KC / 2) % 4 == 2, "row pitches of 2 mod 4 dwords");
    static_assert(lt % 16 == 0 && sc % 16 == 0, "fp32 regions stay 16-byte aligned");
    static_assert(bytes <= 160 * 1024, "LDS of one CU");
};

template <int K, int V, int ACT>
__global__ void __launch_bounds__(kWave * (V / kVW))
__attribute__((amdgpu_waves_per_eu(1, 2)))
gdn_chunk_fwd(const FusedParams p) {
    using Pl = ChunkPlan<K, V, ACT>;
    constexpr int NW = Pl::NW;
    constexpr int P = Pl::P;
    constexpr int KT = Pl::KT;
    constexpr int KC = Pl::KC;
    constexpr int LD = Pl::LD;
    constexpr int KB = K / 32;   // 32-deep steps over the key dimension
    constexpr int MT = K / 16;   // 16-row tiles of the state
    constexpr int CPL = K / 8;   // lanes per token row when staging (8 elements each)
    constexpr int NQK = (kC * CPL + Pl::THREADS - 1) / Pl::THREADS;  // staging vectors per lane
    constexpr uint32_t esz = ACT == 0 ? 4 : 2;

    __shared__ __attribute__((aligned(16))) char smem[Pl::bytes];
    __bf16* const kt = reinterpret_cast<__bf16*>(smem + Pl::kt);
    __bf16* const qt = reinterpret_cast<__bf16*>(smem + Pl::qt);
    __bf16* const kc = reinterpret_cast<__bf16*>(smem + Pl::kc);
    float* const lt = reinterpret_cast<float*>(smem + Pl::lt);
    __bf16* const tb = reinterpret_cast<__bf16*>(smem + Pl::tb);
    __bf16* const pb = reinterpret_cast<__bf16*>(smem + Pl::pb);
    float* const scal = reinterpret_cast<float*>(smem + Pl::sc);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int m16 = lane & 15;   // MFMA row / column of this lane
    const int g4 = lane >> 4;    // MFMA k-group of this lane

    const int seq = blockIdx.x / p.Hv;
    const int h = blockIdx.x % p.Hv;
    const int j = h / p.G;
    const int slot = p.state_idx[seq];
    if (slot < 0) return;  // padding: nothing is read or written
    int64_t bos, eos;
    if (p.cu_seqlens) {
        bos = p.cu_seqlens[seq];
        eos = p.cu_seqlens[seq + 1];
    } else {
        bos = static_cast<int64_t>(seq) * p.T;
        eos = bos + p.T;
    }
    if (eos <= bos) return;
    const int v0 = wave * kVW;
    // Per-lane bases of the A-operand reads: row m16, columns 4 g4 (+16).
    const __bf16* const kt_a = kt + m16 * KT + 4 * g4;
    const __bf16* const qt_a = qt + m16 * KT + 4 * g4;
    const __bf16* const kc_a = kc + m16 * KC + 4 * g4;
    const __bf16* const tb_a = tb + m16 * KC + 4 * g4;
    const __bf16* const pb_a = pb + m16 * KC + 4 * g4;

    // The state slice of this wave: S[mt][ct][r] = S[16 mt + 4 g4 + r][v0 + 16 ct + m16].
    const size_t tile_index = static_cast<size_t>(slot) * p.Hv + h;
    const int sbytes = p.state_bf16 ? 2 : 4;
    const uint32_t row_step = p.state_vk ? 1u : static_cast<uint32_t>(V);   // elements per key row
    const uint32_t col_step = p.state_vk ? static_cast<uint32_t>(K) : 1u;   // elements per value column
    const auto srsrc = buffer_rsrc(static_cast<const char*>(p.pool) + tile_index * K * V * sbytes,
                                   static_cast<uint32_t>(K * V * sbytes));
    // Per-lane byte offset; the rest of each element's offset is uniform.
    const uint32_t s_lane = (4 * g4 * row_step + (v0 + m16) * col_step) * sbytes;
    f32x4 S[MT][kNT];
    if (p.state_bf16) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ct = 0; ct < kNT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S[mt][ct][r] = __uint_as_float(uint32_t(__builtin_amdgcn_raw_buffer_load_b16(
                                                       srsrc, s_lane,
                                                       ((16 * mt + r) * row_step + 16 * ct * col_step) * 2,
                                                       0))
                                                   << 16);
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ct = 0; ct < kNT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S[mt][ct][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        srsrc, s_lane, ((16 * mt + r) * row_step + 16 * ct * col_step) * 4, 0));
    }

    // Activation rows of one chunk are read and written through buffer
    // resources that end after its last token, so rows past the sequence end
    // load as zero and their stores are dropped.
    const uint32_t qrow = static_cast<uint32_t>(p.q_stride) * esz;
    const uint32_t krow = static_cast<uint32_t>(p.k_stride) * esz;
    const uint32_t vrow = static_cast<uint32_t>(p.v_stride) * esz;
    const uint32_t orow = static_cast<uint32_t>(p.Hv) * V * esz;
    const uint32_t act_lane = 4 * g4 * vrow + (v0 + m16) * esz;
    const uint32_t out_lane = 4 * g4 * orow + (v0 + m16) * esz;
    const float A_h = (wave == 0 && !p.g) ? p.A_log[h] : 0.0f;
    const float dtb_h = (wave == 0 && !p.g) ? p.dt_bias[h] : 0.0f;
    const int nchunks = static_cast<int>((eos - bos + kC - 1) / kC);

    auto chunk_len = [&](int cn) {
        const int64_t rest = eos - (bos + static_cast<int64_t>(cn) * kC);
        return static_cast<int>(rest < kC ? rest : kC);
    };
    auto issue_loads = [&](int cn, ChunkLoads<ACT, NQK>& L) {
        const int64_t u0 = bos + static_cast<int64_t>(cn) * kC;
        const int Ln = chunk_len(cn);
        const auto kr = buffer_rsrc(static_cast<const char*>(p.k) + (u0 * p.k_stride + int64_t(j) * K) * esz,
                                    (Ln - 1) * krow + K * esz);
        const auto qr = buffer_rsrc(static_cast<const char*>(p.q) + (u0 * p.q_stride + int64_t(j) * K) * esz,
                                    (Ln - 1) * qrow + K * esz);
        // Vectors past the chunk (vi >= C * CPL, only when the workgroup
        // does not divide the chunk evenly) fall outside the resources and
        // load as zero; there is no branch, so no wait is forced here.
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
            const int vi = tid + i * Pl::THREADS;
            const int t = vi / CPL, c8 = vi % CPL;
#pragma unroll
            for (int h2 = 0; h2 < ChunkLoads<ACT, NQK>::VEC; ++h2) {
                L.k[i][h2] = __builtin_amdgcn_raw_buffer_load_b128(kr, t * krow + (8 * c8 * esz + 16 * h2), 0, 0);
                L.q[i][h2] = __builtin_amdgcn_raw_buffer_load_b128(qr, t * qrow + (8 * c8 * esz + 16 * h2), 0, 0);
            }
        }
        // Gate inputs of token `lane` (wave 0); rows past the chunk load as 0.
        if (wave == 0) {
            if (p.g) {
                const uint32_t grow = static_cast<uint32_t>(p.Hv) * 4;
                const auto gr = buffer_rsrc(p.g + u0 * p.Hv + h, (Ln - 1) * grow + 4);
                const auto br = buffer_rsrc(p.beta + u0 * p.Hv + h, (Ln - 1) * grow + 4);
                L.ga = __builtin_amdgcn_raw_buffer_load_b32(gr, lane * grow, 0, 0);
                L.gb = __builtin_amdgcn_raw_buffer_load_b32(br, lane * grow, 0, 0);
            } else {
                const int64_t e0 = u0 * p.ab_stride + static_cast<int64_t>(h / p.G) * p.ab_khead + h % p.G;
                const uint32_t abrow = static_cast<uint32_t>(p.ab_stride) * esz;
                const auto ar = buffer_rsrc(static_cast<const char*>(p.a) + e0 * esz, (Ln - 1) * abrow + esz);
                const auto br = buffer_rsrc(static_cast<const char*>(p.b) + e0 * esz, (Ln - 1) * abrow + esz);
                if constexpr (ACT == 0) {
                    L.ga = __builtin_amdgcn_raw_buffer_load_b32(ar, lane * abrow, 0, 0);
                    L.gb = __builtin_amdgcn_raw_buffer_load_b32(br, lane * abrow, 0, 0);
                } else {
                    L.ga = __builtin_amdgcn_raw_buffer_load_b16(ar, lane * abrow, 0, 0);
                    L.gb = __builtin_amdgcn_raw_buffer_load_b16(br, lane * abrow, 0, 0);
                }
            }
        }
    };

    // Stage chunk cn from its loads: raw keys and queries into LDS (bf16
    // parts), their inverse norms, the gates and the prefix sums of the
    // log-decays (scalar buffer cn & 1).
    auto stage = [&](int cn, const ChunkLoads<ACT, NQK>& L) {
        const int Ln = chunk_len(cn);
        float* const sc = scal + (cn & 1) * Pl::kScalars * kC;
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
            const int vi = tid + i * Pl::THREADS;
            if ((kC * CPL) % Pl::THREADS == 0 || vi < kC * CPL) {
                const int t = vi / CPL, c8 = vi % CPL;
                float xk[8], xq[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (ACT == 0) {
                        xk[e] = __uint_as_float(L.k[i][0][e]);
                        xk[4 + e] = __uint_as_float(L.k[i][1][e]);
                        xq[e] = __uint_as_float(L.q[i][0][e]);
                        xq[4 + e] = __uint_as_float(L.q[i][1][e]);
                    } else {
                        xk[2 * e] = bf16_lo(L.k[i][0][e]);
                        xk[2 * e + 1] = bf16_hi(L.k[i][0][e]);
                        xq[2 * e] = bf16_lo(L.q[i][0][e]);
                        xq[2 * e + 1] = bf16_hi(L.q[i][0][e]);
                    }
                }
                float ssk = 0.0f, ssq = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ssk = __builtin_fmaf(xk[e], xk[e], ssk);
                    ssq = __builtin_fmaf(xq[e], xq[e], ssq);
                }
                ssk = sum_lane_groups<CPL>(ssk);
                ssq = sum_lane_groups<CPL>(ssq);
                if (c8 == 0) {
                    sc[3 * kC + t] = t < Ln ? rsqrtf(ssk + p.eps) : 0.0f;
                    sc[4 * kC + t] = t < Ln ? p.scale * rsqrtf(ssq + p.eps) : 0.0f;
                }
                if constexpr (ACT == 0) {
                    bf16x8 kh, kl, qh, ql;
                    split8(xk, kh, kl);
                    split8(xq, qh, ql);
                    lds_put8(kt + t * KT + 8 * c8, kh);
                    lds_put8(qt + t * KT + 8 * c8, qh);
                    lds_put8(kt + kC * KT + t * KT + 8 * c8, kl);
                    lds_put8(qt + kC * KT + t * KT + 8 * c8, ql);
                } else {  // bf16 inputs are stored as they came
                    lds_put8(kt + t * KT + 8 * c8, __builtin_bit_cast(bf16x8, L.k[i][0]));
                    lds_put8(qt + t * KT + 8 * c8, __builtin_bit_cast(bf16x8, L.q[i][0]));
                }
            }
        }
        if (wave == 0) {
            float glog, bet;
            if (p.g) {
                glog = __uint_as_float(L.ga);
                bet = __uint_as_float(L.gb);
            } else {
                const uint32_t sh = ACT == 0 ? 0 : 16;   // bf16 in the low half
                gate_values(__uint_as_float(L.ga << sh), __uint_as_float(L.gb << sh), A_h, dtb_h, glog, bet);
            }
            if (lane >= Ln) glog = bet = 0.0f;  // padding tokens: no decay, no update
            const double G = wave_prefix_sum(static_cast<double>(glog));
            const double Glast = readlane_f64(G, kWave - 1);
            // G as an unevaluated float pair: differences of nearby sums then
            // come out exact in the high parts (Sterbenz) plus the low parts
            const float Ghi = static_cast<float>(G);
            sc[lane] = bet;
            sc[5 * kC + lane] = Ghi;
            sc[6 * kC + lane] = static_cast<float>(G - static_cast<double>(Ghi));
            sc[kC + lane] = expf(Ghi);
            sc[2 * kC + lane] = expf(static_cast<float>(Glast - G));
        }
    };

    {
        ChunkLoads<ACT, NQK> ld0;
        issue_loads(0, ld0);
        stage(0, ld0);
    }
    // Past the last chunk the loads and staging below repeat the last
    // chunk's loads (in bounds) and stage into the other scalar buffer and
    // the key/query rows, which nothing reads any more: every iteration then
    // issues the same loads in the same order, and each wait covers exactly
    // the loads it needs.
    const int last = nchunks - 1;
    ChunkLoads<ACT, NQK> ld;
    issue_loads(min(1, last), ld);

    for (int c = 0; c < nchunks; ++c) {
        const int64_t t0 = bos + static_cast<int64_t>(c) * kC;
        const int Lc = chunk_len(c);
        float* const sc = scal + (c & 1) * Pl::kScalars * kC;
        const float* const s_beta = sc;
        const float* const s_eG = sc + kC;
        const float* const s_eGl = sc + 2 * kC;
        const float* const s_rk = sc + 3 * kC;
        const float* const s_rq = sc + 4 * kC;
        const float* const s_G = sc + 5 * kC;
        const float* const s_Glo = sc + 6 * kC;
        lds_barrier();  // chunk c is staged; the previous chunk's products are done
        // This wave's v values (accumulator row order), needed once the
        // state products are done; they land during the Gram tiles.
        float vv[4][kNT][4];
        {
            const auto vr = buffer_rsrc(static_cast<const char*>(p.v) + (t0 * p.v_stride + int64_t(h) * V) * esz,
                                        (Lc - 1) * vrow + V * esz);
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int ct = 0; ct < kNT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t su = (16 * r + e) * vrow + 16 * ct * esz;
                        if constexpr (ACT == 0)
                            vv[r][ct][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vr, act_lane, su, 0));
                        else
                            vv[r][ct][e] = __uint_as_float(
                                uint32_t(__builtin_amdgcn_raw_buffer_load_b16(vr, act_lane, su, 0)) << 16);
                    }
        }

        // ------------------------------------------ B: Gram tiles, D_b = (I + L_bb)^-1
        // 20 tiles: the 4 diagonal blocks of K K^T (then inverted), the 6
        // below them (L), and the 10 of Q K^T on and below the diagonal (P).
        // With 8 wavefronts, wavefronts 4-7 each take one diagonal block,
        // invert it and take one more tile, while wavefronts 0-3 take three
        // tiles each: an inversion costs about as much as two tiles.
        // Otherwise tiles are dealt round-robin.
        auto tile_of = [](int task, bool& isq, int& ti, int& tj) {
            isq = task >= 10;
            if (task < 4) {
                ti = tj = task;
            } else if (!isq) {  // strictly below the diagonal: (1,0),(2,0),(2,1),(3,0),(3,1),(3,2)
                const int o = task - 4;
                ti = o >= 3 ? 3 : o >= 1 ? 2 : 1;
                tj = o - ti * (ti - 1) / 2;
            } else {            // on or below it: (0,0),(1,0),(1,1),(2,0),...,(3,3)
                const int o = task - 10;
                ti = o >= 6 ? 3 : o >= 3 ? 2 : o >= 1 ? 1 : 0;
                tj = o - ti * (ti + 1) / 2;
            }
        };
        // Scales the tile (X K^T)[16 ti.., 16 tj..] held in acc into P (X = Q),
        // the fp32 diagonal block of L, or -L below the diagonal blocks.
        auto tile_epilogue = [&](bool isq, int ti, int tj, const f32x4& acc) {
            // acc[e] = (X K^T)[16 ti + 4 g4 + e][16 tj + m16]
            const int s = 16 * tj + m16;
            const float rks = s_rk[s], Gs = s_G[s], Gls = s_Glo[s];
            const float4 G4 = *reinterpret_cast<const float4*>(s_G + 16 * ti + 4 * g4);
            const float4 GL4 = *reinterpret_cast<const float4*>(s_Glo + 16 * ti + 4 * g4);
            const float4 B4 = *reinterpret_cast<const float4*>(s_beta + 16 * ti + 4 * g4);
            const float4 K4 = *reinterpret_cast<const float4*>(s_rk + 16 * ti + 4 * g4);
            const float4 Q4 = *reinterpret_cast<const float4*>(s_rq + 16 * ti + 4 * g4);
            const float Gt[4] = {G4.x, G4.y, G4.z, G4.w};
            const float GLt[4] = {GL4.x, GL4.y, GL4.z, GL4.w};
            const float Bt[4] = {B4.x * K4.x, B4.y * K4.y, B4.z * K4.z, B4.w * K4.w};
            const float Qt[4] = {Q4.x, Q4.y, Q4.z, Q4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * ti + 4 * g4 + e;
                const float f = t >= s ? expf((Gt[e] - Gs) + (GLt[e] - Gls)) * rks * acc[e] : 0.0f;
                if (isq) {
                    __bf16 hi, lo;
                    split_bf16(Qt[e] * f, hi, lo);
                    pb[t * KC + s] = hi;
                    pb[kC * KC + t * KC + s] = lo;
                } else if (ti == tj) {   // diagonal block of L, fp32, for the inversion
                    lt[(ti * 16 + 4 * g4 + e) * LD + m16] = t > s ? Bt[e] * f : 0.0f;
                } else {                 // -L below the diagonal blocks, for the solve
                    __bf16 hi, lo;
                    split_bf16(-Bt[e] * f, hi, lo);
                    tb[t * KC + s] = hi;
                    tb[kC * KC + t * KC + s] = lo;
                }
            }
        };
        // D_b = (I + L_bb)^-1 from the diagonal block written by this wavefront.
        auto invert_diag = [&](int ti) {
                // D_b = (I + L_bb)^-1 by forward substitution on column m16,
                // four rows at a time: the dot products with the solved rows
                // of earlier quads are split over the four lane groups and
                // summed with two swaps; the quad's own rows follow locally.
                const float* Lb = lt + ti * 16 * LD;
                float y[4] = {0.f, 0.f, 0.f, 0.f};   // y[q] = x[4 q + g4]
#pragma unroll
                for (int pq = 0; pq < 4; ++pq) {
                    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int q = 0; q < pq; ++q)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            part[i] = __builtin_fmaf(Lb[(4 * pq + i) * LD + 4 * q + g4], y[q], part[i]);
                    float xq[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float v = (4 * pq + i == m16 ? 1.0f : 0.0f) - sum_xor32(sum_xor16(part[i]));
#pragma unroll
                        for (int i2 = 0; i2 < i; ++i2)
                            v = __builtin_fmaf(-Lb[(4 * pq + i) * LD + 4 * pq + i2], xq[i2], v);
                        xq[i] = v;
                    }
                    y[pq] = g4 == 0 ? xq[0] : g4 == 1 ? xq[1] : g4 == 2 ? xq[2] : xq[3];
                }
                const int b0 = 16 * ti;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    __bf16 hi, lo;
                    split_bf16(y[q], hi, lo);
                    tb[(b0 + 4 * q + g4) * KC + b0 + m16] = hi;
                    tb[kC * KC + (b0 + 4 * q + g4) * KC + b0 + m16] = lo;
                }
        };
        // (X K^T) tile products on bf16 MFMA (split parts for fp32 inputs).
        auto tile_product = [&](const __bf16* xa, const __bf16* xb, f32x4& acc, int kb) {
            const bf16x8 av = lds_row8_split(xa + 32 * kb);
            const bf16x8 bv = lds_row8_split(xb + 32 * kb);
            acc = mma_bf16(av, bv, acc);
            if constexpr (P == 2) {
                const bf16x8 al = lds_row8_split(xa + kC * KT + 32 * kb);
                const bf16x8 bl = lds_row8_split(xb + kC * KT + 32 * kb);
                acc = mma_bf16(av, bl, acc);
                acc = mma_bf16(al, bv, acc);
            }
        };
        auto gram_tile = [&](int task) {
            bool isq;
            int ti, tj;
            tile_of(task, isq, ti, tj);
            const __bf16* xa = (isq ? qt : kt) + (16 * ti + m16) * KT + 8 * g4;
            const __bf16* xb = kt + (16 * tj + m16) * KT + 8 * g4;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) tile_product(xa, xb, acc, kb);
            tile_epilogue(isq, ti, tj, acc);
            if (task < 4) {
                wave_lds_sync();
                invert_diag(ti);
            }
        };
        if (NW >= 8) {
            // wavefront w < 4: tiles 4+w, 8+w, 12+w; w >= 4: diagonal block
            // w-4, then tile 12+w (16-19)
            const bool inv = wave >= 4;
            const int n = inv ? 2 : 3, step = inv ? 16 : 4;
#pragma unroll 1
            for (int i = 0, task = inv ? wave - 4 : 4 + wave; i < n; ++i, task += step) gram_tile(task);
        } else {
#pragma unroll 1
            for (int task = wave; task < 20; task += NW) gram_tile(task);
        }
        // -------------------------------- C: products with the chunk-start state
        // Keys transposed to [K][C] for the state update (token pairs per lane).
        for (int vi = tid; vi < (kC / 2) * CPL; vi += Pl::THREADS) {
            const int tp = vi % (kC / 2), c8 = vi / (kC / 2);
#pragma unroll
            for (int part = 0; part < P; ++part) {
                const __bf16* src = kt + part * kC * KT + 2 * tp * KT + 8 * c8;
                const bf16x8 a = lds_row8_split(src);
                const bf16x8 b = lds_row8_split(src + KT);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                    bf16x2 w;
                    w[0] = a[e];
                    w[1] = b[e];
                    *reinterpret_cast<bf16x2*>(kc + part * K * KC + (8 * c8 + e) * KC + 2 * tp) = w;
                }
            }
        }
        // KS = K S0 and QS = Q S0 with raw keys and queries.
        f32x4 KS[4][kNT], QS[4][kNT];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int ct = 0; ct < kNT; ++ct) KS[r][ct] = QS[r][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            Split8 so[kNT];
#pragma unroll
            for (int ct = 0; ct < kNT; ++ct) so[ct] = operand_from_tiles(S[2 * kb][ct], S[2 * kb + 1][ct]);
            // all operand reads of this 32-deep step first, so one LDS latency
            // covers the step's 16 products
            bf16x8 ak[4], aq[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                ak[r] = lds_perm8(kt_a + 16 * r * KT + 32 * kb);
                aq[r] = lds_perm8(qt_a + 16 * r * KT + 32 * kb);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int off = 16 * r * KT + 32 * kb;
#pragma unroll
                for (int ct = 0; ct < kNT; ++ct) {
                    KS[r][ct] = mma_bf16(ak[r], so[ct].hi, KS[r][ct]);
                    KS[r][ct] = mma_bf16(ak[r], so[ct].lo, KS[r][ct]);
                    QS[r][ct] = mma_bf16(aq[r], so[ct].hi, QS[r][ct]);
                    QS[r][ct] = mma_bf16(aq[r], so[ct].lo, QS[r][ct]);
                }
                if constexpr (P == 2) {
                    const bf16x8 akl = lds_perm8(kt_a + kC * KT + off);
                    const bf16x8 aql = lds_perm8(qt_a + kC * KT + off);
#pragma unroll
                    for (int ct = 0; ct < kNT; ++ct) {
                        KS[r][ct] = mma_bf16(akl, so[ct].hi, KS[r][ct]);
                        QS[r][ct] = mma_bf16(aql, so[ct].hi, QS[r][ct]);
                    }
                }
            }
        }
        // R = diag(beta) (V - diag(e^G rk) KS) and O = diag(e^G rq) QS.
        f32x4 R[4][kNT], O[4][kNT];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t4 = 16 * r + 4 * g4;
            const float4 b4 = *reinterpret_cast<const float4*>(s_beta + t4);
            const float4 e4 = *reinterpret_cast<const float4*>(s_eG + t4);
            const float4 k4 = *reinterpret_cast<const float4*>(s_rk + t4);
            const float4 q4 = *reinterpret_cast<const float4*>(s_rq + t4);
            const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
            const float ek[4] = {e4.x * k4.x, e4.y * k4.y, e4.z * k4.z, e4.w * k4.w};
            const float eq[4] = {e4.x * q4.x, e4.y * q4.y, e4.z * q4.z, e4.w * q4.w};
#pragma unroll
            for (int ct = 0; ct < kNT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    R[r][ct][e] = bb[e] * (vv[r][ct][e] - ek[e] * KS[r][ct][e]);
                    O[r][ct][e] = eq[e] * QS[r][ct][e];
                }
        }
        lds_barrier();  // D_b, -L, P and the transposed keys are complete

        // The next chunk: stage it (its rows of kt/qt are no longer read) and
        // issue the loads of the one after.
        stage(c + 1, ld);
        issue_loads(min(c + 2, last), ld);

        // --------------------------------------- E: u, outputs, state update
        // U = (I + L)^-1 R by block forward substitution on this wave's
        // columns: U_b = D_b (R_b - sum_{b' < b} L_bb' U_b').
        f32x4 U[4][kNT];
#pragma unroll
        for (int ct = 0; ct < kNT; ++ct) {
            Split4 us[4];
#pragma unroll
            for (int bi = 0; bi < 4; ++bi) {
                // the block row's -L and D_b reads first
                bf16x4 th[4], tl[4];
#pragma unroll
                for (int bj = 0; bj <= bi; ++bj) {
                    th[bj] = *reinterpret_cast<const bf16x4*>(tb_a + 16 * bi * KC + 16 * bj);
                    tl[bj] = *reinterpret_cast<const bf16x4*>(tb_a + kC * KC + 16 * bi * KC + 16 * bj);
                }
                f32x4 acc = R[bi][ct];
#pragma unroll
                for (int bj = 0; bj < bi; ++bj)   // acc += (-L_{bi,bj}) U_bj
                    acc = mma16_split(acc, th[bj], tl[bj], us[bj]);
                const Split4 as = split_tile(acc);
                f32x4 u = {0.f, 0.f, 0.f, 0.f};
                u = mma16_split(u, th[bi], tl[bi], as);
                U[bi][ct] = u;
                us[bi] = split_tile(u);
            }
            // O += P U (P lower triangular, diagonal included); each block
            // row's P reads are issued before its products.
#pragma unroll
            for (int bi = 0; bi < 4; ++bi) {
                bf16x4 ph[4], pl[4];
#pragma unroll
                for (int bj = 0; bj <= bi; ++bj) {
                    ph[bj] = *reinterpret_cast<const bf16x4*>(pb_a + 16 * bi * KC + 16 * bj);
                    pl[bj] = *reinterpret_cast<const bf16x4*>(pb_a + kC * KC + 16 * bi * KC + 16 * bj);
                }
#pragma unroll
                for (int bj = 0; bj <= bi; ++bj) O[bi][ct] = mma16_split(O[bi][ct], ph[bj], pl[bj], us[bj]);
            }
        }
        const auto orr = buffer_rsrc(static_cast<char*>(p.out) + ((t0 * p.Hv + h) * int64_t(V)) * esz,
                                     (Lc - 1) * orow + V * esz);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int ct = 0; ct < kNT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t su = (16 * r + e) * orow + 16 * ct * esz;
                    if constexpr (ACT == 0)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(O[r][ct][e]), orr, out_lane, su, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(bf16_rne(O[r][ct][e])),
                                                              orr, out_lane, su, 0);
                }
        // S' = e^{G_last} S0 + K^T diag(rk e^{G_last - G}) U with raw keys.
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t4 = 16 * r + 4 * g4;
            const float4 k4 = *reinterpret_cast<const float4*>(s_rk + t4);
            const float4 d4 = *reinterpret_cast<const float4*>(s_eGl + t4);
            const float d[4] = {k4.x * d4.x, k4.y * d4.y, k4.z * d4.z, k4.w * d4.w};
#pragma unroll
            for (int ct = 0; ct < kNT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) U[r][ct][e] *= d[e];
        }
        const float eGlast = s_eG[kC - 1];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ct = 0; ct < kNT; ++ct) S[mt][ct] *= eGlast;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            Split8 uo[kNT];
#pragma unroll
            for (int ct = 0; ct < kNT; ++ct) uo[ct] = operand_from_tiles(U[2 * kb][ct], U[2 * kb + 1][ct]);
            bf16x8 ah[MT];   // the step's operand reads first (one LDS latency)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) ah[mt] = lds_perm8(kc_a + 16 * mt * KC + 32 * kb);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int off = 16 * mt * KC + 32 * kb;
#pragma unroll
                for (int ct = 0; ct < kNT; ++ct) {
                    S[mt][ct] = mma_bf16(ah[mt], uo[ct].hi, S[mt][ct]);
                    S[mt][ct] = mma_bf16(ah[mt], uo[ct].lo, S[mt][ct]);
                }
                if constexpr (P == 2) {
                    const bf16x8 al = lds_perm8(kc_a + K * KC + off);
#pragma unroll
                    for (int ct = 0; ct < kNT; ++ct) S[mt][ct] = mma_bf16(al, uo[ct].hi, S[mt][ct]);
                }
            }
        }
    }

    if (!p.write_final) return;
    if (p.state_bf16) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ct = 0; ct < kNT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    __builtin_amdgcn_raw_buffer_store_b16(
                        static_cast<unsigned short>(bf16_rne(S[mt][ct][r])), srsrc, s_lane,
                        ((16 * mt + r) * row_step + 16 * ct * col_step) * 2, 0);
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ct = 0; ct < kNT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    __builtin_amdgcn_raw_buffer_store_b32(
                        __float_as_uint(S[mt][ct][r]), srsrc, s_lane,
                        ((16 * mt + r) * row_step + 16 * ct * col_step) * 4, 0);
    }
}

using ChunkFn = void (*)(FusedParams);

template <int K, int ACT>
ChunkFn chunk_by_v(int V) {
    switch (V) {
        case 32: return &gdn_chunk_fwd<K, 32, ACT>;
        case 64: return &gdn_chunk_fwd<K, 64, ACT>;
        case 128: return &gdn_chunk_fwd<K, 128, ACT>;
        default: return nullptr;
    }
}

template <int ACT>
ChunkFn chunk_by_k(int K, int V) {
    switch (K) {
        case 32: return chunk_by_v<32, ACT>(V);
        case 64: return chunk_by_v<64, ACT>(V);
        case 128: return chunk_by_v<128, ACT>(V);
        default: return nullptr;
    }
}

ChunkFn select_chunk(int K, int V, int act) {
    return act ? chunk_by_k<1>(K, V) : chunk_by_k<0>(K, V);
}

template <int K, int ACT>
int chunk_bytes_by_v(int V) {
    switch (V) {
        case 32: return ChunkPlan<K, 32, ACT>::bytes;
        case 64: return ChunkPlan<K, 64, ACT>::bytes;
        case 128: return ChunkPlan<K, 128, ACT>::bytes;
        default: return 0;
    }
}

}  // namespace

int chunk_block_v() { return kVW; }

int chunk_lds_bytes(int K, int V, int act) {
    if (!select_chunk(K, V, act)) return 0;
    switch (K) {
        case 32: return act ? chunk_bytes_by_v<32, 1>(V) : chunk_bytes_by_v<32, 0>(V);
        case 64: return act ? chunk_bytes_by_v<64, 1>(V) : chunk_bytes_by_v<64, 0>(V);
        case 128: return act ? chunk_bytes_by_v<128, 1>(V) : chunk_bytes_by_v<128, 0>(V);
        default: return 0;
    }
}

hipError_t launch_chunked(const LaunchShape& s, const FusedParams& p, hipStream_t stream) {
    ChunkFn fn = select_chunk(s.K, p.V, s.act);
    if (!fn) return hipErrorInvalidDeviceFunction;
    void* args[] = {const_cast<FusedParams*>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(static_cast<unsigned>(s.groups)),
                           dim3(s.waves * kWave), args, 0, stream);
}

}  // namespace gdn
