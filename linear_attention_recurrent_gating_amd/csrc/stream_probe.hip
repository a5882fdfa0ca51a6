// Memory-stream probes: the state traffic of the decode and spec-verify
// kernels with no arithmetic around it, so that the rate the update kernels
// reach can be put next to the rate the same accesses reach alone.  Built into
// a separate library (libgdn_stream_probe.so) that only the benchmark loads;
// it is not part of the update's C-ABI.
//
// Access shape (the row-split kernel's at K = V = 128 with 32 rows per lane):
// a 256-thread workgroup streams two 64 KiB fp32 tiles, two wavefronts per
// tile.  Lane l of a wavefront covers 16 bytes of row 2i + l/32 of its half of
// the tile, so every 128-bit load or store instruction moves one contiguous
// kilobyte, and each lane issues 32 of them; loads and stores carry the cache
// policies of the update kernels.  Tiles are picked through an index list
// (random slots of a pool, as the decode sees them).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBufNonTemporal = 2;          // loads: "nt"
constexpr int kBufStoreStream = 2 | 16;     // stores: "nt" + "sc1", as the update kernels' state write-back
constexpr int kWord3 = 0x00020000;
constexpr int kTileBytes = 64 * 1024;
constexpr int kRows = 32;            // 128-bit accesses per lane per tile half
constexpr uint32_t kRowStep = 1024;  // bytes between a lane's accesses

enum Kind { kRead = 0, kWrite = 1, kRmw = 2, kCopy = 3, kSpec = 4, kRmwBf16 = 5 };

// bf16 state tiles (32 KiB): the row-split kernel's bf16 access, 8 bytes
// (four elements) per lane, so one 64-bit instruction moves two 256-byte rows;
// 32 of them per lane, two wavefronts per tile, in place.
__global__ void __launch_bounds__(256) gdn_stream_probe_bf16(char* pool, const int32_t* tiles,
                                                             float scale) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    constexpr int kBytes = kTileBytes / 2;
    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    const int64_t slot = static_cast<int64_t>(blockIdx.x) * 2 + wave / 2;
    const int64_t tile = tiles[slot];
    const uint32_t lane_bytes = (wave % 2) * (kBytes / 2) + (lane / 32) * 256 + (lane % 32) * 8;
    const auto r = __builtin_amdgcn_make_buffer_rsrc(pool + tile * kBytes, 0, kBytes, kWord3);
    u32x2 x[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i)
        x[i] = __builtin_amdgcn_raw_buffer_load_b64(r, lane_bytes, i * 512, kBufNonTemporal);
    const uint32_t s = scale == 1.0f ? 0u : 0x00010001u;   // adds nothing unless scale != 1
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        x[i].x += s;
        x[i].y += s;
        __builtin_amdgcn_raw_buffer_store_b64(x[i], r, lane_bytes, i * 512, kBufStoreStream);
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, kTileBytes, kWord3);
}

// tiles[2 b + w/2] is the tile of wavefront w of workgroup b; dst is the
// second buffer (copy: the same tile index there; spec pattern: the four
// intermediate tiles of entry e = i * heads + h go to rows 4 i .. 4 i + 3 of
// an intermediate_states-shaped buffer, tile (4 i + t) * heads + h).
template <int KIND>
__global__ void __launch_bounds__(256) gdn_stream_probe(const char* pool, char* dst,
                                                        const int32_t* tiles, float* sink,
                                                        float scale, int heads) {
    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    const int64_t slot = static_cast<int64_t>(blockIdx.x) * 2 + wave / 2;
    const int64_t tile = tiles[slot];
    const uint32_t lane_bytes = (wave % 2) * (kTileBytes / 2) + (lane / 32) * 512 + (lane % 32) * 16;
    const auto r = rsrc(pool + tile * kTileBytes);
    u32x4 x[kRows];
    if constexpr (KIND != kWrite) {
#pragma unroll
        for (int i = 0; i < kRows; ++i)
            x[i] = __builtin_amdgcn_raw_buffer_load_b128(r, lane_bytes, i * kRowStep, kBufNonTemporal);
    } else {
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const uint32_t s = __float_as_uint(scale * static_cast<float>(i + lane));
            x[i] = u32x4{s, s, s, s};
        }
    }
    if constexpr (KIND == kRead) {
        // every lane stores its sum unconditionally, so no load can be moved
        // under a branch (256 bytes per wavefront against 32 KiB read)
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < kRows; ++i)
            acc += __uint_as_float(x[i].x) + __uint_as_float(x[i].y) + __uint_as_float(x[i].z) +
                   __uint_as_float(x[i].w);
        sink[(static_cast<int64_t>(blockIdx.x) * 4 + wave) * 64 + lane] = acc * scale;
        return;
    } else {
        if constexpr (KIND == kRmw || KIND == kSpec) {
#pragma unroll
            for (int i = 0; i < kRows; ++i)
                x[i] = u32x4{__float_as_uint(__uint_as_float(x[i].x) * scale),
                             __float_as_uint(__uint_as_float(x[i].y) * scale),
                             __float_as_uint(__uint_as_float(x[i].z) * scale),
                             __float_as_uint(__uint_as_float(x[i].w) * scale)};
        }
        if constexpr (KIND == kSpec) {
            const int64_t seq = slot / heads, h = slot % heads;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const auto w = rsrc(dst + ((seq * 4 + t) * heads + h) * kTileBytes);
#pragma unroll
                for (int i = 0; i < kRows; ++i)
                    __builtin_amdgcn_raw_buffer_store_b128(x[i], w, lane_bytes, i * kRowStep, kBufStoreStream);
            }
        }
        const auto w = KIND == kCopy ? rsrc(dst + tile * kTileBytes) : r;
#pragma unroll
        for (int i = 0; i < kRows; ++i)
            __builtin_amdgcn_raw_buffer_store_b128(x[i], w, lane_bytes, i * kRowStep, kBufStoreStream);
    }
}

}  // namespace

extern "C" {

// Streams `num_tiles` (even, > 0) 64 KiB tiles of `pool` chosen by `tiles`
// (device int32 indices) with the access shape above.  kind: 0 read only,
// 1 write only, 2 in-place read-modify-write, 3 copy into `dst` (same tile
// indices), 4 the spec-verify pattern (read once, write four intermediate
// tiles of `dst` laid out as described above for `heads` heads per
// sequence, then write in place; num_tiles a multiple of heads, dst holding
// 4 * num_tiles tiles), 5 in-place read-modify-write of 32 KiB bf16 tiles
// (tile i at byte offset 32 KiB x i of `pool`).  `sink` holds num_tiles *
// 128 floats (read only).  Returns a hipError_t.
int gdn_stream_probe_launch(int kind, const void* pool, void* dst, const int32_t* tiles,
                            int64_t num_tiles, float* sink, float scale, int heads, void* stream) {
    if (num_tiles <= 0 || num_tiles % 2 != 0 || heads <= 0 || num_tiles % heads != 0)
        return static_cast<int>(hipErrorInvalidValue);
    const dim3 grid(static_cast<unsigned>(num_tiles / 2)), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const char* p = static_cast<const char*>(pool);
    char* d = static_cast<char*>(dst);
    switch (kind) {
        case kRead: hipLaunchKernelGGL(gdn_stream_probe<kRead>, grid, block, 0, s, p, d, tiles, sink, scale, heads); break;
        case kWrite: hipLaunchKernelGGL(gdn_stream_probe<kWrite>, grid, block, 0, s, p, d, tiles, sink, scale, heads); break;
        case kRmw: hipLaunchKernelGGL(gdn_stream_probe<kRmw>, grid, block, 0, s, p, d, tiles, sink, scale, heads); break;
        case kCopy: hipLaunchKernelGGL(gdn_stream_probe<kCopy>, grid, block, 0, s, p, d, tiles, sink, scale, heads); break;
        case kSpec: hipLaunchKernelGGL(gdn_stream_probe<kSpec>, grid, block, 0, s, p, d, tiles, sink, scale, heads); break;
        case kRmwBf16: hipLaunchKernelGGL(gdn_stream_probe_bf16, grid, block, 0, s, const_cast<char*>(p), tiles, scale); break;
        default: return static_cast<int>(hipErrorInvalidValue);
    }
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
