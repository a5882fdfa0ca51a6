// State-tile streaming and q/k staging shared by the per-token kernels
// (column tiles, row split, value rows).  Device code only.
#pragma once

#include "gdn_device.h"

namespace gdn {
namespace {

constexpr int kMaxThreads = 512;

// The state streams through HBM once per call (read, then written back), so
// its loads and stores carry the non-temporal hint.  They are raw buffer
// operations on a resource that spans exactly one K x V tile: the tile base
// sits in SGPRs, each lane keeps one 32-bit byte offset in a VGPR, and the
// row-group step is a scalar offset -- no 64-bit address per row stays live
// between the loads and the final stores.  Offsets past the tile would be
// clamped by the hardware (loads return 0, stores are dropped).  Tiles may be
// stored as bf16 (64-bit accesses per four elements, rounded to nearest even
// on the way out); the state is fp32 in registers either way.

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One K x V state tile in the pool or in intermediate_states, stored as fp32
// or as bf16 (the arithmetic is fp32 either way).  Offsets are in elements;
// `lane` is this lane's element offset within the tile.
struct TileIO {
    __amdgpu_buffer_rsrc_t r;
    uint32_t lane_bytes;
    bool bf16;
};

__device__ __forceinline__ TileIO tile_io(const void* base, bool bf16, size_t tile_index,
                                          size_t tile_elems, uint32_t lane) {
    const int sh = bf16 ? 1 : 2;
    const char* b = static_cast<const char*>(base) + ((tile_index * tile_elems) << sh);
    TileIO t;
    t.r = buffer_rsrc(b, static_cast<uint32_t>(tile_elems << sh));
    t.lane_bytes = lane << sh;
    t.bf16 = bf16;
    return t;
}

// Issues the loads of N groups of four consecutive state elements, group i at
// element offset off(i) past the lane's, as raw words (fp32: four words; bf16:
// two words in .x/.y).  One branch on the storage type covers all N loads, so
// none waits for another; tile_unpack, placed at the first use, waits for them.
template <int N, typename OFF>
__device__ __forceinline__ void tile_issue(const TileIO& t, OFF off, u32x4 (&raw)[N]) {
    if (t.bf16) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(t.r, t.lane_bytes, off(i) << 1,
                                                                 kBufNonTemporal);
            raw[i].x = v[0];
            raw[i].y = v[1];
        }
    } else {
        // 16 idle cycles between the 1 KiB fp32 loads of a wavefront: measured
        // on MI355X against back-to-back issue, the bs=512 decode takes 352.7
        // vs 355.5 us and the spec-verify batch 282 vs 286 us (other
        // wavefronts' accesses interleave instead of queueing behind a burst).
#pragma unroll
        for (int i = 0; i < N; ++i) {
            raw[i] = __builtin_amdgcn_raw_buffer_load_b128(t.r, t.lane_bytes, off(i) << 2, kBufNonTemporal);
            asm volatile("s_nop 7\n\ts_nop 7");
        }
    }
}

// Widens raw words from tile_issue to fp32 (bf16 -> fp32 is exact).
template <int N>
__device__ __forceinline__ void tile_unpack(bool bf16, const u32x4 (&raw)[N], float4 (&s)[N]) {
    if (bf16) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            s[i] = make_float4(__uint_as_float(raw[i].x << 16), __uint_as_float(raw[i].x & 0xffff0000u),
                               __uint_as_float(raw[i].y << 16), __uint_as_float(raw[i].y & 0xffff0000u));
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i)
            s[i] = make_float4(__uint_as_float(raw[i].x), __uint_as_float(raw[i].y),
                               __uint_as_float(raw[i].z), __uint_as_float(raw[i].w));
    }
}

// Stores N groups of four state elements (group i at element offset off(i)
// past the lane's), rounding to bf16 (nearest even) for bf16 storage.
template <int N, typename OFF>
__device__ __forceinline__ void tile_store_all(const TileIO& t, OFF off, const float4 (&s)[N]) {
    if (t.bf16) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const u32x2 v = {bf16_rne_pair(s[i].x, s[i].y), bf16_rne_pair(s[i].z, s[i].w)};
            __builtin_amdgcn_raw_buffer_store_b64(v, t.r, t.lane_bytes, off(i) << 1, kBufStoreStream);
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const u32x4 v = {__float_as_uint(s[i].x), __float_as_uint(s[i].y), __float_as_uint(s[i].z),
                             __float_as_uint(s[i].w)};
            __builtin_amdgcn_raw_buffer_store_b128(v, t.r, t.lane_bytes, off(i) << 2, kBufStoreStream);
        }
    }
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

}  // namespace
}  // namespace gdn
