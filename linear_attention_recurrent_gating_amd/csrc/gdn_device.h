// Device helpers shared by the HIP kernels of libgdn: activation loads and
// stores, bf16 rounding, cross-lane sums, the LDS barrier and the gates.
// Private to the library (each translation unit gets its own copy).
#pragma once

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kWave = 64;

// Raw buffer resources: the base sits in SGPRs and each lane supplies a 32-bit
// byte offset.  Accesses at or past `bytes` are bounds-checked by the hardware
// (loads return 0, stores are dropped).
constexpr int kBufNonTemporal = 2;           // cache-policy bit "nt" (gfx94x/gfx950)
// State write-back: "nt" plus "sc1" (device scope).  On MI355X a probe of the
// decode's in-place tile stream (1 GiB of 64 KiB tiles at random slots) ran
// at 344.5 us with it against 350.0 us with "nt" alone, and write-only
// streams 2% faster; loads keep "nt" (with "sc1" they ran no faster).
constexpr int kBufStoreStream = 2 | 16;
// Word 3 of a gfx9-family raw buffer resource: 32-bit data format, no swizzle.
constexpr int kBufWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                             kBufWord3);
}

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN); on gfx950
// the conversion is v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two values rounded to bf16 and packed (the first in the low half): one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t bf16_rne_pair(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) { return bf16_rne(f); }

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
        w.x = bf16_rne_pair(o.x, o.y);
        w.y = bf16_rne_pair(o.z, o.w);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + e) = w;
    }
}

// One output element (bf16 rounded to nearest even).
template <int ACT>
__device__ __forceinline__ void store1_act(void* base, int64_t e, float o) {
    if constexpr (ACT == 0) static_cast<float*>(base)[e] = o;
    else static_cast<uint16_t*>(base)[e] = static_cast<uint16_t>(bf16_rne(o));
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

// Sum over aligned groups of N consecutive lanes (N = 2..64), leaving every
// lane of a group with a bitwise identical sum: quad swaps, the half-row and
// row mirrors, then the permlane16/32 swaps.  Each step pairs lanes that
// already hold identical partial sums, and fp32 addition is commutative.
template <int N>
__device__ __forceinline__ float sum_lane_groups(float x) {
    static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "power-of-two group");
    if constexpr (N >= 2) x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
    if constexpr (N >= 4) x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
    if constexpr (N >= 8) x += dpp_mov<0x141>(x);   // row_half_mirror
    if constexpr (N >= 16) x += dpp_mov<0x140>(x);  // row_mirror
    if constexpr (N >= 32) x = sum_xor16(x);
    if constexpr (N >= 64) x = sum_xor32(x);
    return x;
}

// Returns x unchanged but hidden from the optimiser, so that values derived
// from it (per-row buffer offsets) are formed where they are used instead of
// being hoisted out of a loop and kept live in scalar registers across it.
__device__ __forceinline__ uint32_t opaque_uniform(uint32_t x) {
    asm volatile("" : "+s"(x));
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
// g = -exp(A_log) * softplus(a + dt_bias) (the log-decay), beta = sigmoid(b).
// softplus returns x itself above 20, where log1p(exp(x)) - x < 2.1e-9.
__device__ __forceinline__ void gate_values(float a, float b, float A_log, float dt_bias,
                                            float& g, float& beta) {
    const float x = a + dt_bias;
    const float sp = x > 20.0f ? x : log1pf(expf(x));
    g = -expf(A_log) * sp;
    beta = 1.0f / (1.0f + expf(-b));
}

// The log-decay g and beta of token t, v-head h: computed from a and b
// (element t*ab_stride + (h/G)*ab_khead + h%G, which also reads a/b packed per
// k-head), or taken from precomputed g and beta ([N, H_v] fp32, the unfused
// pair).  Both routes give the same fp32 g.  A_log and dt_bias are read only
// on the fused route (they may be null with precomputed gates).
template <int ACT>
__device__ __forceinline__ void token_log_gate(const FusedParams& p, int64_t t, int h, float& g,
                                               float& beta) {
    if (p.g) {
        g = p.g[t * p.Hv + h];
        beta = p.beta[t * p.Hv + h];
    } else {
        const int64_t e = t * p.ab_stride + static_cast<int64_t>(h / p.G) * p.ab_khead + h % p.G;
        gate_values(load_scalar<ACT>(p.a, e), load_scalar<ACT>(p.b, e), p.A_log[h], p.dt_bias[h],
                    g, beta);
    }
}

// The decay factor gamma = exp(g) and beta of token t, v-head h.
template <int ACT>
__device__ __forceinline__ void token_gates(const FusedParams& p, int64_t t, int h, float& gamma,
                                            float& beta) {
    float g;
    token_log_gate<ACT>(p, t, h, g, beta);
    gamma = expf(g);
}

}  // namespace
}  // namespace gdn
