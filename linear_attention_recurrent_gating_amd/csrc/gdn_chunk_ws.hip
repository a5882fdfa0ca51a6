// Chunked forward of the gated delta rule in two passes over a workspace.
//
// The chunk algebra is the WY form written out at the top of gdn_chunk.hip:
// for one (sequence, v-head) and one chunk of 64 tokens with start state S0,
//   U  = (I + L)^-1 R,      R = diag(beta) (V - diag(e^G rk) K S0)
//   O  = diag(e^G rq) Q S0 + P U
//   S' = e^{G_last} S0 + K^T diag(rk e^{G_last - G}) U
// with L[t][s] = beta_t e^{G_t-G_s} rk_t rk_s (k_t . k_s) for s < t and
// P[t][s] = rq_t rk_s e^{G_t-G_s} (q_t . k_s) for s <= t (K, Q raw rows).
// Everything except R, U, O and S' is independent of the state.  sglang PR
// #21411 (implementation section) builds these per-chunk matrices -- the key
// Gram product and the triangular solve -- in a kernel of their own that runs
// over all chunks at once (with a chunk index table for varlen batches), and
// leaves the sequential pass over the chunks to a second kernel.  Here:
//
//   gdn_chunk_prep   one workgroup per (chunk slot, k-head), all in parallel:
//                    the Gram tiles on bf16 MFMA once for the k-head, then
//                    per v-head the scaled L and P, the full inverse
//                    A = (I + L)^-1 (diagonal blocks by forward substitution,
//                    the blocks below them on fp32 MFMA), and the per-token
//                    scalars.  A and P are written as the bf16 hi/lo operand
//                    fragments the state pass reads.
//   gdn_chunk_state  one workgroup per (sequence, v-head), eight wavefronts of
//                    16 value columns with their K x 16 state slice in MFMA
//                    accumulators, walking the chunks in order: K S0 and Q S0,
//                    U = A R (four independent block rows rather than a
//                    dependent substitution), O and S'.
//
// Chunk slots.  Chunk c of sequence i goes to slot floor(bos_i / 64) + i + c.
// Slots of different (sequence, chunk) pairs differ, because a sequence of
// L tokens starting at bos spans at most floor((bos mod 64 + L) / 64) + 1
// slots before the next sequence's first one; the largest slot is below
// floor(N / 64) + B.  The prep kernel finds the sequence of its slot by a
// 64-way search over the (strictly increasing) slot bases, so no index table
// has to be built first; slots that belong to no chunk exit at once.
//
// Precision.  As in gdn_chunk.hip: raw bf16 keys and queries are exact MFMA
// operands, fp32 operands are split into bf16 hi + lo parts (three
// products), the log-decay prefix sums are taken in fp64 and kept as a float
// pair.  The off-diagonal blocks of (I + L)^-1 are products of fp32 blocks on
// the fp32 matrix instructions.  With bf16 activations, the two products that
// feed only the output (Q S0 and P U) take the hi parts alone: the output is
// rounded to bf16 (8 significant bits) anyway, and every product that feeds
// the state keeps its split operands.

#include "gdn_chunk_common.h"

namespace gdn {
namespace {

constexpr int kBlk = 10;                 // lower-triangular 16 x 16 blocks of a 64 x 64 matrix
constexpr int kFragBytes = 64 * 4 * 2;   // one bf16x4 operand fragment per lane
constexpr int kWsScalars = 5;            // beta, e^G rk, e^G rq, rk e^{G_last - G}, e^{G_last}

// One workspace entry: the state pass's operands for one (chunk slot, v-head).
struct WsEntry {
    static constexpr int A = 0;                              // (I + L)^-1: [block][hi, lo][lane][4]
    static constexpr int P = A + kBlk * 2 * kFragBytes;      // P, same layout
    static constexpr int SC = P + kBlk * 2 * kFragBytes;     // [kWsScalars][64] fp32
    static constexpr int bytes = SC + kWsScalars * kC * 4;
};
static_assert(WsEntry::bytes % 256 == 0, "entries stay 256-byte aligned");
static_assert(WsEntry::bytes % 16 == 0, "entries are copied as 16-byte vectors");

__device__ __forceinline__ int blk_of(int bi, int bj) { return bi * (bi + 1) / 2 + bj; }

__device__ __forceinline__ int64_t seq_bos(const FusedParams& p, int i) {
    return p.cu_seqlens ? static_cast<int64_t>(p.cu_seqlens[i]) : static_cast<int64_t>(i) * p.T;
}
__device__ __forceinline__ int64_t seq_eos(const FusedParams& p, int i) {
    return p.cu_seqlens ? static_cast<int64_t>(p.cu_seqlens[i + 1]) : static_cast<int64_t>(i + 1) * p.T;
}
// First chunk slot of sequence i.
__device__ __forceinline__ int64_t slot_base(const FusedParams& p, int i) {
    return seq_bos(p, i) / kC + i;
}

// The largest i in [0, B) whose first slot is <= w (every lane gets it).
// Each round probes 64 evenly spaced candidates and keeps the interval after
// the last one that qualifies; slot bases increase strictly with i.
__device__ int find_seq(const FusedParams& p, int B, int64_t w, int lane) {
    int lo = 0, n = B;
    while (n > 1) {
        const int step = (n + kWave - 1) / kWave;
        const int off = lane * step;
        const bool ok = off < n && slot_base(p, lo + off) <= w;
        const uint64_t m = __builtin_amdgcn_ballot_w64(ok);
        const int last = 63 - __builtin_clzll(m);   // lane 0 always qualifies
        lo += last * step;
        n = min(step, n - last * step);
    }
    return lo;
}

// fp32 16 x 16 x 16 product on v_mfma_f32_16x16x4_f32: acc += X Y for X, Y
// row-major 16 x 16 fp32 blocks in LDS (pitch LDB).  Lane (g, m) supplies
// X[m][4 kb + g] and Y[4 kb + g][m]; acc[r] is row 4 g + r, column m.
template <int LDB>
__device__ __forceinline__ f32x4 block_mul_f32(const float* X, const float* Y, f32x4 acc, int g4,
                                               int m16) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[m16 * LDB + 4 * kb + g4], Y[(4 * kb + g4) * LDB + m16],
                                                   acc, 0, 0, 0);
    return acc;
}

template <int K, int ACT>
struct PrepPlan {
    static constexpr int THREADS = 256;
    static constexpr int P = ACT == 0 ? 2 : 1;   // bf16 parts per input element
    // Pitch of the staged [C][K] rows (bf16).  The Gram operands are 16-byte
    // reads, lane (g, m) taking row m at dword 4 g; on gfx950 that pattern
    // runs at 256 B/clk per CU with a pitch of 8 mod 16 dwords and at 157
    // B/clk with one of 4 mod 8 (measured with 8 wavefronts per CU).  The
    // staging writes whole rows, which no pitch makes conflict.
    static constexpr int KT = K + 16;
    static constexpr int LDB = 18;               // pitch of a 16 x 16 fp32 block (8-byte rows)
    static constexpr int BLK = 16 * LDB;         // floats per block
    static constexpr int stage_bytes = 2 * P * kC * KT * 2;
    static constexpr int block_bytes = 2 * kBlk * BLK * 4;   // L, A (fp32)
    static constexpr int r0 = 0;                  // staged keys/queries, then the fp32 blocks
    static constexpr int r0_bytes = stage_bytes > block_bytes ? stage_bytes : block_bytes;
    static constexpr int kBatch = 4;              // v-heads whose gates are prepared at once
    static constexpr int sc = r0 + r0_bytes;      // rk, rq: [2][C]; then beta, G hi, G lo: [3][kBatch][C]
    static constexpr int bytes = sc + (2 + 3 * kBatch) * kC * 4;
    static_assert((KT / 2) % 16 == 8 && (KT * 2) % 16 == 0, "16-byte rows, pitch 8 mod 16 dwords");
    static_assert(ACT == 0 || bytes <= 40 * 1024, "four prep workgroups per CU (bf16 inputs)");
    static_assert(bytes <= 80 * 1024, "two prep workgroups per CU (fp32 inputs)");
};

// Per (chunk slot, k-head): L, P and (I + L)^-1 of the chunk for each of the
// k-head's G v-heads, packed into their workspace entries.  The keys and
// queries are staged and their Gram tiles computed once; the gates, scaling
// and inversion are per v-head.  Four wavefronts.
template <int K, int ACT>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(ACT == 0 ? 2 : 4, 4)))   // the workgroups per CU the LDS allows
gdn_chunk_prep(const FusedParams p, char* ws, int B) {
    using Pl = PrepPlan<K, ACT>;
    constexpr int P = Pl::P;
    constexpr int KT = Pl::KT;
    constexpr int LDB = Pl::LDB;
    constexpr int BLK = Pl::BLK;
    constexpr int KB = K / 32;
    constexpr int CPL = K / 8;                                   // lanes per staged row
    constexpr int NQK = (kC * CPL + Pl::THREADS - 1) / Pl::THREADS;
    constexpr uint32_t esz = ACT == 0 ? 4 : 2;

    __shared__ __attribute__((aligned(16))) char smem[Pl::bytes];
    __bf16* const kt = reinterpret_cast<__bf16*>(smem + Pl::r0);
    __bf16* const qt = kt + P * kC * KT;
    float* const Lb = reinterpret_cast<float*>(smem + Pl::r0);  // after the Gram tiles
    float* const Ab = Lb + kBlk * BLK;
    float* const s_rk = reinterpret_cast<float*>(smem + Pl::sc);
    float* const s_rq = s_rk + kC;
    float* const s_beta0 = s_rq + kC;                  // [kBatch][C] each
    float* const s_G0 = s_beta0 + Pl::kBatch * kC;
    float* const s_Glo0 = s_G0 + Pl::kBatch * kC;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int m16 = lane & 15;
    const int g4 = lane >> 4;

    const int64_t w = blockIdx.x / p.Hk;
    const int j = static_cast<int>(blockIdx.x % p.Hk);
    int32_t slot;
    int64_t bos, eos;
    int i;
    if (B <= kWave) {
        // one round trip: lane l loads sequence l's bounds and slot index, the
        // sequence of this chunk slot is the last whose first slot is <= w
        const int l = lane < B ? lane : 0;
        const int32_t slot_l = p.state_idx[l];
        const int64_t bos_l = seq_bos(p, l), eos_l = seq_eos(p, l);
        const uint64_t m = __builtin_amdgcn_ballot_w64(lane < B && bos_l / kC + l <= w);
        i = 63 - __builtin_clzll(m);   // lane 0 always qualifies
        slot = __builtin_amdgcn_readlane(slot_l, i);
        bos = readlane_i64(bos_l, i);
        eos = readlane_i64(eos_l, i);
    } else {
        i = find_seq(p, B, w, lane);
        // the slot index and the sequence bounds load together
        slot = p.state_idx[i];
        bos = seq_bos(p, i);
        eos = seq_eos(p, i);
    }
    if (slot < 0) return;
    const int64_t c = w - (bos / kC + i);
    const int64_t t0 = bos + c * kC;
    if (t0 >= eos) return;   // a slot past the sequence's last chunk: no chunk
    const int Lc = static_cast<int>(eos - t0 < kC ? eos - t0 : kC);

    // Gate inputs of token `lane` for v-head g of the group, and that head's
    // A_log and dt_bias: wave w prepares v-heads w, w + 4, ... (one batch of
    // four v-heads at a time), its first ones loaded ahead of the key/query
    // rows so that the latencies overlap.
    float ga_n = 0.0f, gb_n = 0.0f, Alog_n = 0.0f, dtb_n = 0.0f;
    auto load_gates = [&](int g) {
        ga_n = gb_n = 0.0f;
        if (g < p.G) {
            if (!p.g) {
                Alog_n = p.A_log[j * p.G + g];
                dtb_n = p.dt_bias[j * p.G + g];
            }
            if (lane < Lc) {
                const int64_t t = t0 + lane;
                if (p.g) {
                    const int h = j * p.G + g;
                    ga_n = p.g[t * p.Hv + h];
                    gb_n = p.beta[t * p.Hv + h];
                } else {
                    const int64_t e = t * p.ab_stride + static_cast<int64_t>(j) * p.ab_khead + g;
                    ga_n = load_scalar<ACT>(p.a, e);
                    gb_n = load_scalar<ACT>(p.b, e);
                }
            }
        }
    };
    load_gates(wave);

    // Gates and log-decay prefix sums of v-head gb + wave (token `lane`) into
    // the batch's LDS scalars, and the state pass's per-token scalars of that
    // head: beta and e^{G_last} at once, the three that need the norms from
    // e^G and e^{G_last - G}, kept in registers until the norms are staged.
    float eG_w = 0.0f, dG_w = 0.0f;
    auto sc_of = [&](int g) {
        return reinterpret_cast<float*>(ws + (static_cast<size_t>(w) * p.Hv + j * p.G + g) * WsEntry::bytes +
                                        WsEntry::SC);
    };
    auto gate_prep = [&](int gb) {
        if (gb + wave < p.G) {
            float glog = 0.0f, bet = 0.0f;
            if (lane < Lc) {
                if (p.g) {
                    glog = ga_n;
                    bet = gb_n;
                } else {
                    gate_values(ga_n, gb_n, Alog_n, dtb_n, glog, bet);
                }
            }
            load_gates(gb + wave + Pl::kBatch);   // the next batch's, ahead
            const double G = wave_prefix_sum(static_cast<double>(glog));
            // G as an unevaluated float pair: differences of nearby sums come
            // out exact in the high parts (Sterbenz) plus the low parts
            const float Ghi = static_cast<float>(G);
            s_beta0[wave * kC + lane] = bet;
            s_G0[wave * kC + lane] = Ghi;
            s_Glo0[wave * kC + lane] = static_cast<float>(G - static_cast<double>(Ghi));
            const double Glast = readlane_f64(G, kWave - 1);
            float* const out_sc = sc_of(gb + wave);
            out_sc[lane] = bet;
            out_sc[4 * kC + lane] = exp_hw(static_cast<float>(Glast));
            eG_w = exp_hw(Ghi);
            dG_w = exp_hw(static_cast<float>(Glast - G));
        }
    };
    auto write_scalars = [&](int gb) {
        if (gb + wave < p.G) {
            float* const out_sc = sc_of(gb + wave);
            const float rk = s_rk[lane], rq = s_rq[lane];
            out_sc[kC + lane] = eG_w * rk;
            out_sc[2 * kC + lane] = eG_w * rq;
            out_sc[3 * kC + lane] = rk * dG_w;
        }
    };

    // ---- stage raw keys and queries (rows past the chunk load as zero) and
    // their inverse norms
    {
        const uint32_t krow = static_cast<uint32_t>(p.k_stride) * esz;
        const uint32_t qrow = static_cast<uint32_t>(p.q_stride) * esz;
        const auto kr = buffer_rsrc(static_cast<const char*>(p.k) + (t0 * p.k_stride + int64_t(j) * K) * esz,
                                    (Lc - 1) * krow + K * esz);
        const auto qr = buffer_rsrc(static_cast<const char*>(p.q) + (t0 * p.q_stride + int64_t(j) * K) * esz,
                                    (Lc - 1) * qrow + K * esz);
        static_assert((kC * CPL) % Pl::THREADS == 0, "whole rows per pass");
        // every row load first (one round trip), as raw words, then the norms
        // and (fp32 inputs) the splits; bf16 rows are staged as loaded
        constexpr int VEC = ACT == 0 ? 2 : 1;
        u32x4v rks_[NQK][VEC], rqs_[NQK][VEC];
#pragma unroll
        for (int n = 0; n < NQK; ++n) {
            const int vi = tid + n * Pl::THREADS;
            const int t = vi / CPL, c8 = vi % CPL;
#pragma unroll
            for (int h2 = 0; h2 < VEC; ++h2) {
                rks_[n][h2] = __builtin_amdgcn_raw_buffer_load_b128(kr, t * krow + 8 * c8 * esz + 16 * h2, 0, 0);
                rqs_[n][h2] = __builtin_amdgcn_raw_buffer_load_b128(qr, t * qrow + 8 * c8 * esz + 16 * h2, 0, 0);
            }
        }
        // the first batch's gates while the rows are in flight
        gate_prep(0);
        auto widen8 = [](const u32x4v (&w)[VEC], float (&x)[8]) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (ACT == 0) {
                    x[e] = __uint_as_float(w[0][e]);
                    x[4 + e] = __uint_as_float(w[VEC - 1][e]);
                } else {
                    x[2 * e] = bf16_lo(w[0][e]);
                    x[2 * e + 1] = bf16_hi(w[0][e]);
                }
            }
        };
#pragma unroll
        for (int n = 0; n < NQK; ++n) {
            const int vi = tid + n * Pl::THREADS;
            const int t = vi / CPL, c8 = vi % CPL;
            float xk[8], xq[8];
            widen8(rks_[n], xk);
            widen8(rqs_[n], xq);
            float ssk = 0.0f, ssq = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ssk = __builtin_fmaf(xk[e], xk[e], ssk);
                ssq = __builtin_fmaf(xq[e], xq[e], ssq);
            }
            ssk = sum_lane_groups<CPL>(ssk);
            ssq = sum_lane_groups<CPL>(ssq);
            if (c8 == 0) {
                s_rk[t] = t < Lc ? rsqrtf(ssk + p.eps) : 0.0f;
                s_rq[t] = t < Lc ? p.scale * rsqrtf(ssq + p.eps) : 0.0f;
            }
            if constexpr (ACT == 0) {
                bf16x8 kh, kl, qh, ql;
                split8(xk, kh, kl);
                split8(xq, qh, ql);
                *reinterpret_cast<bf16x8*>(kt + t * KT + 8 * c8) = kh;
                *reinterpret_cast<bf16x8*>(qt + t * KT + 8 * c8) = qh;
                *reinterpret_cast<bf16x8*>(kt + kC * KT + t * KT + 8 * c8) = kl;
                *reinterpret_cast<bf16x8*>(qt + kC * KT + t * KT + 8 * c8) = ql;
            } else {
                *reinterpret_cast<u32x4v*>(kt + t * KT + 8 * c8) = rks_[n][0];
                *reinterpret_cast<u32x4v*>(qt + t * KT + 8 * c8) = rqs_[n][0];
            }
        }
    }
    lds_barrier();

    // ---- raw Gram tiles, once for the group: task 0..3 the diagonal blocks
    // of K K^T, 4..9 the blocks below them, 10..19 the blocks of Q K^T on and
    // below the diagonal, those computed transposed (K Q^T): the accumulator
    // of a transposed tile holds in lane (g, m) row m and columns 4 g .. + 3
    // of the Q K^T block, which is the operand fragment the state pass reads,
    // so P goes from registers to the workspace without passing through LDS.
    auto tile_of = [](int task, bool& isq, int& ti, int& tj) {
        isq = task >= 10;
        if (task < 4) {
            ti = tj = task;
        } else if (!isq) {
            const int o = task - 4;
            ti = o >= 3 ? 3 : o >= 1 ? 2 : 1;
            tj = o - ti * (ti - 1) / 2;
        } else {
            const int o = task - 10;
            ti = o >= 6 ? 3 : o >= 3 ? 2 : o >= 1 ? 1 : 0;
            tj = o - ti * (ti + 1) / 2;
        }
    };
    f32x4 acc[5];
#pragma unroll
    for (int n = 0; n < 5; ++n) {
        bool isq;
        int ti, tj;
        tile_of(wave + 4 * n, isq, ti, tj);
        const __bf16* xa = kt + (16 * (isq ? tj : ti) + m16) * KT + 8 * g4;
        const __bf16* xb = (isq ? qt : kt) + (16 * (isq ? ti : tj) + m16) * KT + 8 * g4;
        acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const bf16x8 av = lds_row8(xa + 32 * kb);
            const bf16x8 bv = lds_row8(xb + 32 * kb);
            acc[n] = mma_bf16(av, bv, acc[n]);
            if constexpr (P == 2) {
                const bf16x8 al = lds_row8(xa + kC * KT + 32 * kb);
                const bf16x8 bl = lds_row8(xb + kC * KT + 32 * kb);
                acc[n] = mma_bf16(av, bl, acc[n]);
                acc[n] = mma_bf16(al, bv, acc[n]);
            }
        }
    }
    // (the barrier at the top of the v-head loop ends the staged rows' life:
    // the region then holds L and A)

#pragma unroll 1
    for (int gb = 0; gb < p.G; gb += Pl::kBatch) {
        // ---- the batch's gates (the first batch's were prepared during the
        // staging) and the state pass's per-token scalars of its heads
        if (gb > 0) gate_prep(gb);
        write_scalars(gb);
        lds_barrier();   // this batch's gates are in; the staged rows are dead

#pragma unroll 1
    for (int g = gb; g < p.G && g < gb + Pl::kBatch; ++g) {
        const int h = j * p.G + g;
        char* const entry = ws + (static_cast<size_t>(w) * p.Hv + h) * WsEntry::bytes;
        const float* const s_beta = s_beta0 + (g - gb) * kC;
        const float* const s_G = s_G0 + (g - gb) * kC;
        const float* const s_Glo = s_Glo0 + (g - gb) * kC;
        if (g > gb) lds_barrier();   // the previous v-head's blocks are packed

        // ---- scale into L (strictly below the diagonal; LDS) and P (on and
        // below it; straight into the entry's operand fragments)
#pragma unroll
        for (int n = 0; n < 5; ++n) {
            bool isq;
            int ti, tj;
            tile_of(wave + 4 * n, isq, ti, tj);
            if (!isq) {
                // L block (ti, tj): lane (g, m) holds rows t = 16 ti + 4 g + e,
                // column s = 16 tj + m
                const int s = 16 * tj + m16;
                const float rks = s_rk[s], Gs = s_G[s], Gls = s_Glo[s];
                const int t4 = 16 * ti + 4 * g4;
                const float4 G4 = *reinterpret_cast<const float4*>(s_G + t4);
                const float4 GL4 = *reinterpret_cast<const float4*>(s_Glo + t4);
                const float4 X4 = *reinterpret_cast<const float4*>(s_beta + t4);
                const float4 K4 = *reinterpret_cast<const float4*>(s_rk + t4);
                const float Gt[4] = {G4.x, G4.y, G4.z, G4.w};
                const float GLt[4] = {GL4.x, GL4.y, GL4.z, GL4.w};
                const float Xt[4] = {X4.x, X4.y, X4.z, X4.w};
                const float Kt[4] = {K4.x, K4.y, K4.z, K4.w};
                float* const dst = Lb + blk_of(ti, tj) * BLK;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = t4 + e;
                    // (computed for every element, kept below the diagonal)
                    const float ex = exp_hw((Gt[e] - Gs) + (GLt[e] - Gls));
                    dst[(4 * g4 + e) * LDB + m16] = t > s ? Xt[e] * Kt[e] * (ex * rks * acc[n][e]) : 0.0f;
                }
            } else {
                // P block (ti, tj), transposed tile: lane (g, m) holds row
                // t = 16 ti + m, columns s = 16 tj + 4 g + e
                const int t = 16 * ti + m16;
                const float rqt = s_rq[t], Gt = s_G[t], Glt = s_Glo[t];
                const int s4 = 16 * tj + 4 * g4;
                const float4 G4 = *reinterpret_cast<const float4*>(s_G + s4);
                const float4 GL4 = *reinterpret_cast<const float4*>(s_Glo + s4);
                const float4 K4 = *reinterpret_cast<const float4*>(s_rk + s4);
                const float Gs[4] = {G4.x, G4.y, G4.z, G4.w};
                const float GLs[4] = {GL4.x, GL4.y, GL4.z, GL4.w};
                const float Ks[4] = {K4.x, K4.y, K4.z, K4.w};
                f32x4 pv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = s4 + e;
                    const float ex = exp_hw((Gt - Gs[e]) + (Glt - GLs[e]));
                    pv[e] = t >= s ? rqt * (ex * Ks[e] * acc[n][e]) : 0.0f;
                }
                const Split4 sp = split_tile(pv);
                char* const base = entry + WsEntry::P + blk_of(ti, tj) * 2 * kFragBytes + lane * 8;
                *reinterpret_cast<bf16x4*>(base) = sp.hi;
                if constexpr (P == 2)   // with bf16 activations the state pass reads P's hi parts only
                    *reinterpret_cast<bf16x4*>(base + kFragBytes) = sp.lo;
            }
        }
        lds_barrier();

        // ---- D_b = (I + L_bb)^-1 by forward substitution on column m16, four
        // rows per round (wave b takes diagonal block b)
        {
            const int b = wave;
            const float* Lbb = Lb + blk_of(b, b) * BLK;
            float y[4] = {0.f, 0.f, 0.f, 0.f};   // y[q] = D[4 q + g4][m16]
#pragma unroll
            for (int pq = 0; pq < 4; ++pq) {
                float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < pq; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        part[r] = __builtin_fmaf(Lbb[(4 * pq + r) * LDB + 4 * q + g4], y[q], part[r]);
                float xq[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = (4 * pq + r == m16 ? 1.0f : 0.0f) - sum_xor32(sum_xor16(part[r]));
#pragma unroll
                    for (int r2 = 0; r2 < r; ++r2)
                        v = __builtin_fmaf(-Lbb[(4 * pq + r) * LDB + 4 * pq + r2], xq[r2], v);
                    xq[r] = v;
                }
                y[pq] = g4 == 0 ? xq[0] : g4 == 1 ? xq[1] : g4 == 2 ? xq[2] : xq[3];
            }
            float* const Dbb = Ab + blk_of(b, b) * BLK;
#pragma unroll
            for (int q = 0; q < 4; ++q) Dbb[(4 * q + g4) * LDB + m16] = y[q];
        }
        lds_barrier();

        // ---- blocks below the diagonal: A_ij = -D_i sum_{k=j}^{i-1} L_ik A_kj,
        // by distance i - j (three rounds; wave n takes block (n + d, n))
#pragma unroll
        for (int d = 1; d <= 3; ++d) {
            if (wave < 4 - d) {
                const int bi = wave + d, bj = wave;
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < d; ++k)
                    x = block_mul_f32<LDB>(Lb + blk_of(bi, bj + k) * BLK, Ab + blk_of(bj + k, bj) * BLK, x, g4,
                                           m16);
                float* const Aij = Ab + blk_of(bi, bj) * BLK;   // holds X until D_i X replaces it
#pragma unroll
                for (int r = 0; r < 4; ++r) Aij[(4 * g4 + r) * LDB + m16] = x[r];
                wave_lds_sync();
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
                a = block_mul_f32<LDB>(Ab + blk_of(bi, bi) * BLK, Aij, a, g4, m16);
                wave_lds_sync();
#pragma unroll
                for (int r = 0; r < 4; ++r) Aij[(4 * g4 + r) * LDB + m16] = -a[r];
            }
            lds_barrier();
        }

        // ---- pack A into bf16 hi/lo operand fragments: lane (g, m) of
        // block (bi, bj) holds rows 16 bi + m, columns 16 bj + 4 g .. + 3
#pragma unroll
        for (int n = 0; n < 3; ++n) {
            const int blk = wave + 4 * n;
            if (blk < kBlk) {
                const float* const src = Ab + blk * BLK + m16 * LDB + 4 * g4;
                const float2 v01 = *reinterpret_cast<const float2*>(src);
                const float2 v23 = *reinterpret_cast<const float2*>(src + 2);
                const Split4 sp = split_tile(f32x4{v01.x, v01.y, v23.x, v23.y});
                char* const base = entry + WsEntry::A + blk * 2 * kFragBytes + lane * 8;
                *reinterpret_cast<bf16x4*>(base) = sp.hi;
                *reinterpret_cast<bf16x4*>(base + kFragBytes) = sp.lo;
            }
        }
    }
    }
}

// Per (sequence, v-head): the state pass over the chunks, reading each
// chunk's A, P and scalars from the workspace.  Each wavefront holds one
// 16-column tile of the state.  (Two tiles per wavefront, so that every
// operand fragment read from LDS serves both, halved the LDS traffic but left
// one wavefront per SIMD at V = 128 with nothing to hide its latencies behind:
// 166 against 133 us on the long varlen batch.)
template <int K, int V, int ACT>
struct StatePlan {
    static constexpr int NW = V / 16;
    static constexpr int THREADS = NW * kWave;
    static constexpr int P = ACT == 0 ? 2 : 1;
    // Row pitches of 2 mod 4 dwords: the 16 lanes that one cycle of an 8-byte
    // operand read serves (rows m16 = 0..15 at one column) then fall on 16
    // distinct bank pairs.  (At a pitch of 0 mod 4 dwords rows m16 and m16 + 8
    // share banks: the operand reads, pairs of 8-byte reads 32 bytes apart,
    // measured 156 B/clk per CU at 2 mod 4 and 85 at 4 mod 8.)  Rows are
    // therefore only 8-byte aligned, and every access to them is 8 bytes wide
    // at most.
    static constexpr int KT = K + 4;              // pitch of [C][K] (bf16)
    static constexpr int KC = kC + 4;             // pitch of [K][C] (bf16)
    static constexpr int kt = 0;                                  // P x [C][KT] raw keys
    static constexpr int qt = kt + P * kC * KT * 2;               // P x [C][KT] raw queries
    static constexpr int kc = qt + P * kC * KT * 2;               // P x [K][KC] raw keys, transposed
    static constexpr int en = (kc + P * K * KC * 2 + 15) / 16 * 16;   // the chunk's workspace entry
    static constexpr int bytes = en + WsEntry::bytes;
    static constexpr int EV = WsEntry::bytes / 16;                // 16-byte vectors per entry
    static constexpr int NEV = (EV + THREADS - 1) / THREADS;      // per thread
    static_assert(V % 16 == 0 && K % 32 == 0, "16-column waves, 32-deep key steps");
    static_assert((KT / 2) % 4 == 2 && (KC / 2) % 4 == 2, "row pitches of 2 mod 4 dwords");
    static_assert(bytes <= 160 * 1024, "LDS of one CU");
};

template <int K, int V, int ACT>
__global__ void __launch_bounds__(kWave * (V / 16))
__attribute__((amdgpu_waves_per_eu(1, 2)))
gdn_chunk_state(const FusedParams p, const char* ws) {
    using Pl = StatePlan<K, V, ACT>;
    constexpr int P = Pl::P;
    constexpr int KT = Pl::KT;
    constexpr int KC = Pl::KC;
    constexpr int KB = K / 32;
    constexpr int MT = K / 16;
    constexpr int CPL = K / 8;
    constexpr int NQK = (kC * CPL + Pl::THREADS - 1) / Pl::THREADS;
    constexpr int VEC = ACT == 0 ? 2 : 1;
    constexpr uint32_t esz = ACT == 0 ? 4 : 2;

    __shared__ __attribute__((aligned(16))) char smem[Pl::bytes];
    __bf16* const kt = reinterpret_cast<__bf16*>(smem + Pl::kt);
    __bf16* const qt = reinterpret_cast<__bf16*>(smem + Pl::qt);
    __bf16* const kc = reinterpret_cast<__bf16*>(smem + Pl::kc);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int m16 = lane & 15;
    const int g4 = lane >> 4;

    const int seq = blockIdx.x / p.Hv;
    const int h = blockIdx.x % p.Hv;
    const int j = h / p.G;
    const int slot = p.state_idx[seq];
    if (slot < 0) return;
    const int64_t bos = seq_bos(p, seq), eos = seq_eos(p, seq);
    if (eos <= bos) return;
    const int64_t sbase = slot_base(p, seq);
    const int nchunks = static_cast<int>((eos - bos + kC - 1) / kC);
    const int v0 = wave * 16;
    const __bf16* const kt_a = kt + m16 * KT + 4 * g4;
    const __bf16* const qt_a = qt + m16 * KT + 4 * g4;
    const __bf16* const kc_a = kc + m16 * KC + 4 * g4;

    // The state slice of this wave: S[mt][r] = S[16 mt + 4 g4 + r][v0 + m16].
    const size_t tile_index = static_cast<size_t>(slot) * p.Hv + h;
    const int sbytes = p.state_bf16 ? 2 : 4;
    const uint32_t row_step = p.state_vk ? 1u : static_cast<uint32_t>(V);
    const uint32_t col_step = p.state_vk ? static_cast<uint32_t>(K) : 1u;
    const auto srsrc = buffer_rsrc(static_cast<const char*>(p.pool) + tile_index * K * V * sbytes,
                                   static_cast<uint32_t>(K * V * sbytes));
    const uint32_t s_lane = (4 * g4 * row_step + (v0 + m16) * col_step) * sbytes;
    f32x4 S[MT];
    if (p.state_bf16) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[mt][r] = __uint_as_float(uint32_t(__builtin_amdgcn_raw_buffer_load_b16(
                                               srsrc, s_lane, ((16 * mt + r) * row_step) * 2, 0))
                                           << 16);
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[mt][r] = __uint_as_float(
                    __builtin_amdgcn_raw_buffer_load_b32(srsrc, s_lane, ((16 * mt + r) * row_step) * 4, 0));
    }

    const uint32_t qrow = static_cast<uint32_t>(p.q_stride) * esz;
    const uint32_t krow = static_cast<uint32_t>(p.k_stride) * esz;
    const uint32_t vrow = static_cast<uint32_t>(p.v_stride) * esz;
    const uint32_t orow = static_cast<uint32_t>(p.Hv) * V * esz;
    const uint32_t act_lane = 4 * g4 * vrow + (v0 + m16) * esz;
    const uint32_t out_lane = 4 * g4 * orow + (v0 + m16) * esz;

    auto chunk_len = [&](int cn) {
        const int64_t rest = eos - (bos + static_cast<int64_t>(cn) * kC);
        return static_cast<int>(rest < kC ? rest : kC);
    };
    // Token t and 8-element column group c8 that thread-slot vi stages.  At
    // K = 128 each 16 lanes take 8 groups of two tokens (rather than all 16
    // groups of one), so that their 8-byte LDS writes cover all 32 banks
    // once; every 8 lanes still load 128 contiguous bytes of a row.
    auto stage_pos = [](int vi, int& t, int& c8) {
        if constexpr (CPL == 16) {
            const int r = vi % 32;
            t = 2 * (vi / 32) + ((r >> 3) & 1);
            c8 = (r & 7) + 8 * (r >> 4);
        } else {
            t = vi / CPL;
            c8 = vi % CPL;
        }
    };
    // Loads of one chunk, issued a chunk ahead: raw keys and queries, and the
    // chunk's workspace entry.
    struct Loads {
        u32x4v k[NQK][VEC];
        u32x4v q[NQK][VEC];
        u32x4v e[Pl::NEV];
    };
    auto issue_loads = [&](int cn, Loads& L) {
        const int64_t u0 = bos + static_cast<int64_t>(cn) * kC;
        const int Ln = chunk_len(cn);
        const auto kr = buffer_rsrc(static_cast<const char*>(p.k) + (u0 * p.k_stride + int64_t(j) * K) * esz,
                                    (Ln - 1) * krow + K * esz);
        const auto qr = buffer_rsrc(static_cast<const char*>(p.q) + (u0 * p.q_stride + int64_t(j) * K) * esz,
                                    (Ln - 1) * qrow + K * esz);
#pragma unroll
        for (int n = 0; n < NQK; ++n) {
            int t, c8;
            stage_pos(tid + n * Pl::THREADS, t, c8);
#pragma unroll
            for (int h2 = 0; h2 < VEC; ++h2) {
                L.k[n][h2] = __builtin_amdgcn_raw_buffer_load_b128(kr, t * krow + (8 * c8 * esz + 16 * h2), 0, 0);
                L.q[n][h2] = __builtin_amdgcn_raw_buffer_load_b128(qr, t * qrow + (8 * c8 * esz + 16 * h2), 0, 0);
            }
        }
        const auto er = buffer_rsrc(ws + ((sbase + cn) * p.Hv + h) * static_cast<int64_t>(WsEntry::bytes),
                                    WsEntry::bytes);
#pragma unroll
        for (int n = 0; n < Pl::NEV; ++n)   // vectors past the entry load as zero
            L.e[n] = __builtin_amdgcn_raw_buffer_load_b128(er, (tid + n * Pl::THREADS) * 16, 0, 0);
    };
    // Raw keys and queries into kt/qt (bf16 parts), the entry into its buffer.
    auto stage = [&](int cn, const Loads& L) {
#pragma unroll
        for (int n = 0; n < NQK; ++n) {
            const int vi = tid + n * Pl::THREADS;
            if ((kC * CPL) % Pl::THREADS == 0 || vi < kC * CPL) {
                int t, c8;
                stage_pos(vi, t, c8);
                if constexpr (ACT == 0) {
                    float xk[8], xq[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        xk[e] = __uint_as_float(L.k[n][e / 4][e % 4]);
                        xq[e] = __uint_as_float(L.q[n][e / 4][e % 4]);
                    }
                    bf16x8 kh, kl, qh, ql;
                    split8(xk, kh, kl);
                    split8(xq, qh, ql);
                    lds_put8(kt + t * KT + 8 * c8, kh);
                    lds_put8(qt + t * KT + 8 * c8, qh);
                    lds_put8(kt + kC * KT + t * KT + 8 * c8, kl);
                    lds_put8(qt + kC * KT + t * KT + 8 * c8, ql);
                } else {
                    lds_put8(kt + t * KT + 8 * c8, __builtin_bit_cast(bf16x8, L.k[n][0]));
                    lds_put8(qt + t * KT + 8 * c8, __builtin_bit_cast(bf16x8, L.q[n][0]));
                }
            }
        }
        char* const eb = smem + Pl::en;
#pragma unroll
        for (int n = 0; n < Pl::NEV; ++n) {
            const int vi = tid + n * Pl::THREADS;
            if (Pl::EV % Pl::THREADS == 0 || vi < Pl::EV) *reinterpret_cast<u32x4v*>(eb + vi * 16) = L.e[n];
        }
    };
    // Keys transposed to [K][C] (token pairs per lane) from the staged rows.
    auto transpose_keys = [&]() {
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
                    bf16x2 w2;
                    w2[0] = a[e];
                    w2[1] = b[e];
                    *reinterpret_cast<bf16x2*>(kc + part * K * KC + (8 * c8 + e) * KC + 2 * tp) = w2;
                }
            }
        }
    };

    // This wave's v values of chunk cn (accumulator row order) as raw words;
    // rows past the chunk load as zero.  They are widened where they are
    // used, in the next iteration: a widening here, next to the loads, would
    // make the wave wait for them, and for the prefetches issued after them,
    // at the end of this iteration.
    auto load_v = [&](int cn, uint32_t (&vraw)[4][4]) {
        const int64_t u0 = bos + static_cast<int64_t>(cn) * kC;
        const auto vr = buffer_rsrc(static_cast<const char*>(p.v) + (u0 * p.v_stride + int64_t(h) * V) * esz,
                                    (chunk_len(cn) - 1) * vrow + V * esz);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t su = (16 * r + e) * vrow;
                if constexpr (ACT == 0)
                    vraw[r][e] = __builtin_amdgcn_raw_buffer_load_b32(vr, act_lane, su, 0);
                else
                    vraw[r][e] = __builtin_amdgcn_raw_buffer_load_b16(vr, act_lane, su, 0);
            }
    };
    auto v_value = [](uint32_t raw) { return __uint_as_float(ACT == 0 ? raw : raw << 16); };

    // Past the last chunk the loads below repeat the last chunk's (in bounds,
    // unused), so that every iteration issues the same loads in the same
    // order and each wait covers exactly the loads it needs.
    const int last = nchunks - 1;
    Loads ld;
    issue_loads(0, ld);
    stage(0, ld);
    uint32_t vraw[4][4];
    load_v(0, vraw);
    issue_loads(min(1, last), ld);

    for (int c = 0; c < nchunks; ++c) {
        const int64_t t0 = bos + static_cast<int64_t>(c) * kC;
        const int Lc = chunk_len(c);
        // Every read of the staged entry comes before this chunk's second
        // barrier, after which the next chunk's entry is staged over it.
        const char* const eb = smem + Pl::en;
        const float* const s_beta = reinterpret_cast<const float*>(eb + WsEntry::SC);
        const float* const s_ek = s_beta + kC;
        const float* const s_eq = s_beta + 2 * kC;
        const float* const s_d = s_beta + 3 * kC;
        lds_barrier();   // chunk c is staged; chunk c - 1's key transpose is read
        const float eGlast = s_beta[4 * kC];
        transpose_keys();   // read only by this chunk's state update, after the next barrier

        // KS = K S0 and QS = Q S0 with raw keys and queries.
        f32x4 KS[4], QS[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) KS[r] = QS[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const Split8 so = operand_from_tiles(S[2 * kb], S[2 * kb + 1]);
            bf16x8 ak[4], aq[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                ak[r] = lds_perm8(kt_a + 16 * r * KT + 32 * kb);
                aq[r] = lds_perm8(qt_a + 16 * r * KT + 32 * kb);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                KS[r] = mma_bf16(ak[r], so.hi, KS[r]);
                KS[r] = mma_bf16(ak[r], so.lo, KS[r]);
                QS[r] = mma_bf16(aq[r], so.hi, QS[r]);
                if constexpr (P == 2)   // bf16 outputs: the hi part of S0 suffices
                    QS[r] = mma_bf16(aq[r], so.lo, QS[r]);
                if constexpr (P == 2) {
                    const int off = 16 * r * KT + 32 * kb;
                    KS[r] = mma_bf16(lds_perm8(kt_a + kC * KT + off), so.hi, KS[r]);
                    QS[r] = mma_bf16(lds_perm8(qt_a + kC * KT + off), so.hi, QS[r]);
                }
            }
        }
        // R = diag(beta) (V - diag(e^G rk) KS), split for the products with A;
        // O starts as diag(e^G rq) QS.
        Split4 rs[4];
        f32x4 O[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t4 = 16 * r + 4 * g4;
            const float4 b4 = *reinterpret_cast<const float4*>(s_beta + t4);
            const float4 k4 = *reinterpret_cast<const float4*>(s_ek + t4);
            const float4 q4 = *reinterpret_cast<const float4*>(s_eq + t4);
            const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
            const float ek[4] = {k4.x, k4.y, k4.z, k4.w};
            const float eq[4] = {q4.x, q4.y, q4.z, q4.w};
            f32x4 R;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                R[e] = bb[e] * (v_value(vraw[r][e]) - ek[e] * KS[r][e]);
                O[r][e] = eq[e] * QS[r][e];
            }
            rs[r] = split_tile(R);
        }
        // U = A R: the four block rows are independent.
        const char* const fa = eb + WsEntry::A + lane * 8;
        const char* const fp = eb + WsEntry::P + lane * 8;
        f32x4 U[4];
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
            bf16x4 ah[4], al[4];
#pragma unroll
            for (int bj = 0; bj <= bi; ++bj) {
                ah[bj] = *reinterpret_cast<const bf16x4*>(fa + blk_of(bi, bj) * 2 * kFragBytes);
                al[bj] = *reinterpret_cast<const bf16x4*>(fa + blk_of(bi, bj) * 2 * kFragBytes + kFragBytes);
            }
            f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int bj = 0; bj <= bi; ++bj) u = mma16_split(u, ah[bj], al[bj], rs[bj]);
            U[bi] = u;
        }
        // O += P U (P lower triangular, diagonal included).
        Split4 us[4];
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) us[bj] = split_tile(U[bj]);
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
            bf16x4 ph[4], pl[4];
#pragma unroll
            for (int bj = 0; bj <= bi; ++bj) {
                ph[bj] = *reinterpret_cast<const bf16x4*>(fp + blk_of(bi, bj) * 2 * kFragBytes);
                if constexpr (P == 2)
                    pl[bj] = *reinterpret_cast<const bf16x4*>(fp + blk_of(bi, bj) * 2 * kFragBytes + kFragBytes);
            }
#pragma unroll
            for (int bj = 0; bj <= bi; ++bj) {
                if constexpr (P == 2)
                    O[bi] = mma16_split(O[bi], ph[bj], pl[bj], us[bj]);
                else   // bf16 outputs: single bf16 operands
                    O[bi] = mma16(ph[bj], us[bj].hi, O[bi]);
            }
        }
        const auto orr = buffer_rsrc(static_cast<char*>(p.out) + ((t0 * p.Hv + h) * int64_t(V)) * esz,
                                     (Lc - 1) * orow + V * esz);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t su = (16 * r + e) * orow;
                if constexpr (ACT == 0)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(O[r][e]), orr, out_lane, su, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(bf16_rne(O[r][e])), orr,
                                                          out_lane, su, 0);
            }
        // U rows scaled by rk e^{G_last - G} for the state update.
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float4 d4 = *reinterpret_cast<const float4*>(s_d + 16 * r + 4 * g4);
            U[r][0] *= d4.x;
            U[r][1] *= d4.y;
            U[r][2] *= d4.z;
            U[r][3] *= d4.w;
        }
        lds_barrier();   // kt/qt and the entry are read; the key transpose is complete

        // The next chunk: stage its rows and entry, load its v (this chunk's
        // are consumed; issued first, so that waiting for them never waits
        // for the loads after), and issue the loads of the chunk after it.
        // After the last chunk the staged rows and entry are never read.
        stage(c + 1, ld);
        load_v(min(c + 1, last), vraw);
        issue_loads(min(c + 2, last), ld);

        // S' = e^{G_last} S0 + K^T diag(rk e^{G_last - G}) U with raw keys.
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) S[mt] *= eGlast;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const Split8 uo = operand_from_tiles(U[2 * kb], U[2 * kb + 1]);
            bf16x8 ah[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) ah[mt] = lds_perm8(kc_a + 16 * mt * KC + 32 * kb);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                S[mt] = mma_bf16(ah[mt], uo.hi, S[mt]);
                S[mt] = mma_bf16(ah[mt], uo.lo, S[mt]);
                if constexpr (P == 2)
                    S[mt] = mma_bf16(lds_perm8(kc_a + K * KC + 16 * mt * KC + 32 * kb), uo.hi, S[mt]);
            }
        }
    }

    if (!p.write_final) return;
    if (p.state_bf16) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(bf16_rne(S[mt][r])), srsrc,
                                                      s_lane, ((16 * mt + r) * row_step) * 2, 0);
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[mt][r]), srsrc, s_lane,
                                                      ((16 * mt + r) * row_step) * 4, 0);
    }
}

using PrepFn = void (*)(FusedParams, char*, int);
using StateFn = void (*)(FusedParams, const char*);

template <int ACT>
PrepFn prep_by_k(int K) {
    switch (K) {
        case 32: return &gdn_chunk_prep<32, ACT>;
        case 64: return &gdn_chunk_prep<64, ACT>;
        case 128: return &gdn_chunk_prep<128, ACT>;
        default: return nullptr;
    }
}

template <int K, int ACT>
StateFn state_by_v(int V) {
    switch (V) {
        case 32: return &gdn_chunk_state<K, 32, ACT>;
        case 64: return &gdn_chunk_state<K, 64, ACT>;
        case 128: return &gdn_chunk_state<K, 128, ACT>;
        default: return nullptr;
    }
}

template <int ACT>
StateFn state_by_k(int K, int V) {
    switch (K) {
        case 32: return state_by_v<32, ACT>(V);
        case 64: return state_by_v<64, ACT>(V);
        case 128: return state_by_v<128, ACT>(V);
        default: return nullptr;
    }
}

}  // namespace

int64_t chunk_ws_entry_bytes() { return WsEntry::bytes; }

int64_t chunk_ws_slots(int64_t num_tokens, int num_seqs) { return num_tokens / kC + num_seqs; }

hipError_t launch_chunked_ws(const LaunchShape& s, const FusedParams& p, int num_seqs,
                             int64_t num_tokens, void* workspace, hipStream_t stream) {
    PrepFn prep = s.act ? prep_by_k<1>(s.K) : prep_by_k<0>(s.K);
    StateFn state = s.act ? state_by_k<1>(s.K, p.V) : state_by_k<0>(s.K, p.V);
    if (!prep || !state) return hipErrorInvalidDeviceFunction;
    const int64_t prep_groups = chunk_ws_slots(num_tokens, num_seqs) * p.Hk;
    if (prep_groups > INT32_MAX) return hipErrorInvalidConfiguration;
    char* ws = static_cast<char*>(workspace);
    {
        int b = num_seqs;
        void* args[] = {const_cast<FusedParams*>(&p), &ws, &b};
        const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(prep),
                                             dim3(static_cast<unsigned>(prep_groups)), dim3(256), args, 0,
                                             stream);
        if (e != hipSuccess) return e;
    }
    const char* cws = ws;
    void* args[] = {const_cast<FusedParams*>(&p), &cws};
    return hipLaunchKernel(reinterpret_cast<const void*>(state), dim3(static_cast<unsigned>(s.groups)),
                           dim3(s.waves * kWave), args, 0, stream);
}

}  // namespace gdn
