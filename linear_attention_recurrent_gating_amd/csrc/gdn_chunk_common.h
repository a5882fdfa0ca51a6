// Matrix-core helpers shared by the chunked forward kernels (gdn_chunk.hip:
// one workgroup per (sequence, v-head) building every matrix itself;
// gdn_chunk_ws.hip: a pre-pass over all chunks plus a state pass).  Device
// code only.
#pragma once

#include "gdn_device.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

constexpr int kC = 64;           // tokens per chunk

__device__ __forceinline__ f32x4 mma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// x = hi + lo + O(2^-17 |x|), both parts bf16 (round to nearest even).
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
    hi = static_cast<__bf16>(x);
    lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

// split_bf16 of a pair, bit for bit: each part of the pair is one packed
// conversion (v_cvt_pk_bf16_f32), and the hi parts are widened back from the
// packed word (a shift and a mask): 3 VALU instructions per element where
// converting element by element and then packing takes 4.
__device__ __forceinline__ void split_bf16x2(float a, float b, bf16x2& hi, bf16x2& lo) {
    hi = __builtin_convertvector(f32x2{a, b}, bf16x2);
    const uint32_t w = __builtin_bit_cast(uint32_t, hi);
    lo = __builtin_convertvector(f32x2{a - __uint_as_float(w << 16), b - __uint_as_float(w & 0xffff0000u)},
                                 bf16x2);
}

// split_bf16 of eight elements.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
    bf16x2 h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split_bf16x2(x[2 * i], x[2 * i + 1], h[i], l[i]);
    hi = __builtin_shufflevector(__builtin_shufflevector(h[0], h[1], 0, 1, 2, 3),
                                 __builtin_shufflevector(h[2], h[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
    lo = __builtin_shufflevector(__builtin_shufflevector(l[0], l[1], 0, 1, 2, 3),
                                 __builtin_shufflevector(l[2], l[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x16_bf16: A[m][4 g + i] and B[4 g + i][n] in lane (g, m / n);
// the accumulator layout of a 16-row tile is exactly its B-operand layout.
__device__ __forceinline__ f32x4 mma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                      __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

struct Split4 {
    bf16x4 hi, lo;
};

__device__ __forceinline__ Split4 split_tile(const f32x4& x) {
    bf16x2 h0, l0, h1, l1;
    split_bf16x2(x[0], x[1], h0, l0);
    split_bf16x2(x[2], x[3], h1, l1);
    Split4 r;
    r.hi = __builtin_shufflevector(h0, h1, 0, 1, 2, 3);
    r.lo = __builtin_shufflevector(l0, l1, 0, 1, 2, 3);
    return r;
}

// acc += A X for a 16 x 16 block A given as bf16 hi/lo parts (this lane's
// four elements, read from LDS by the caller ahead of the products) and X a
// 16-row accumulator tile of this lane split the same way: hi*hi + hi*lo +
// lo*hi.
__device__ __forceinline__ f32x4 mma16_split(f32x4 acc, const bf16x4& ah, const bf16x4& al,
                                             const Split4& x) {
    acc = mma16(ah, x.hi, acc);
    acc = mma16(ah, x.lo, acc);
    acc = mma16(al, x.hi, acc);
    return acc;
}

struct Split8 {
    bf16x8 hi, lo;
};

// The B operand of one 32-deep step taken from two 16-row accumulator tiles
// of this lane: element e < 4 is row 4*(lane/16) + e of tile a, element e >= 4
// row 4*(lane/16) + e - 4 of tile b.
__device__ __forceinline__ Split8 operand_from_tiles(const f32x4& a, const f32x4& b) {
    const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    Split8 r;
    split8(x, r.hi, r.lo);
    return r;
}

// The matching A operand: elements p[0..3] and p[16..19] of an LDS row.
__device__ __forceinline__ bf16x8 lds_perm8(const __bf16* p) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 16);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Eight consecutive bf16 of an LDS row (16-byte aligned).
__device__ __forceinline__ bf16x8 lds_row8(const __bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

// Eight bf16 into a row that is only 8-byte aligned: two 8-byte writes.
__device__ __forceinline__ void lds_put8(__bf16* dst, const bf16x8& x) {
    *reinterpret_cast<bf16x4*>(dst) = __builtin_shufflevector(x, x, 0, 1, 2, 3);
    *reinterpret_cast<bf16x4*>(dst + 4) = __builtin_shufflevector(x, x, 4, 5, 6, 7);
}

// The same from a row that is only 8-byte aligned: two 8-byte reads.
__device__ __forceinline__ bf16x8 lds_row8_split(const __bf16* p) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 4);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Eight consecutive activation elements at byte offset `off`, widened to fp32.
template <int ACT>
__device__ __forceinline__ void buffer_load8(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&x)[8]) {
    if constexpr (ACT == 0) {
        const u32x4v a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        const u32x4v b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = __uint_as_float(a[e]);
            x[4 + e] = __uint_as_float(b[e]);
        }
    } else {
        const u32x4v a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = bf16_lo(a[e]);
            x[2 * e + 1] = bf16_hi(a[e]);
        }
    }
}

// Inclusive prefix sum over the 64 lanes: a Hillis-Steele scan inside each
// 16-lane row (row_shr 1, 2, 4, 8; lanes shifted in from outside the row add
// 0), then the row totals carried down with row_bcast:15 and row_bcast:31.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or_zero(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, true));
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_or_zero(double v) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        0, static_cast<int>(static_cast<uint32_t>(b)), CTRL, ROW_MASK, 0xF, true));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        0, static_cast<int>(static_cast<uint32_t>(b >> 32)), CTRL, ROW_MASK, 0xF, true));
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// In fp64: the chunk's log-decay prefix sums can reach thousands when a
// token's gate saturates, and the Gram scaling needs exp(G_t - G_s) for
// neighbouring tokens, a small difference of two large sums.
__device__ __forceinline__ double wave_prefix_sum(double x) {
    x += dpp_or_zero<0x111, 0xF>(x);  // row_shr:1
    x += dpp_or_zero<0x112, 0xF>(x);  // row_shr:2
    x += dpp_or_zero<0x114, 0xF>(x);  // row_shr:4
    x += dpp_or_zero<0x118, 0xF>(x);  // row_shr:8
    x += dpp_or_zero<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_or_zero<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

__device__ __forceinline__ double readlane_f64(double x, int l) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(x));
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(b)), l));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(b >> 32)), l));
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// e^x on the hardware base-2 exponential (v_exp_f32, about one ulp) of
// x log2(e).  Rounding that product adds a relative error of about
// |x| 2^-24 (below 1e-6 for |x| <= 16); the chunk's decay factors
// e^{G_t - G_s} it serves lie in (0, 1], and where |x| is larger they are
// negligible beside the factors near 1.  Overflows to +inf above x = 88.7,
// as expf does; no denormal or special-case handling beyond the
// instruction's own.
__device__ __forceinline__ float exp_hw(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

__device__ __forceinline__ int64_t readlane_i64(int64_t x, int l) {
    const uint64_t b = static_cast<uint64_t>(x);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(b)), l));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(b >> 32)), l));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// LDS written by some lanes of this wavefront becomes visible to its others.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Staging loads of one chunk, issued a chunk ahead so that they land while
// the previous chunk's products run: raw keys and queries (16-byte vectors,
// NQK per lane) and the raw gate inputs of token `lane` (wave 0).
// The gate inputs stay raw words until staging (a bf16 value in the low
// half): widening them next to their loads would make the wave wait there
// for every load issued before, the key/query prefetch included.
template <int ACT, int NQK>
struct ChunkLoads {
    static constexpr int VEC = ACT == 0 ? 2 : 1;   // 16-byte vectors per 8 elements
    u32x4v k[NQK][VEC];
    u32x4v q[NQK][VEC];
    uint32_t ga, gb;
};

}  // namespace
}  // namespace gdn
