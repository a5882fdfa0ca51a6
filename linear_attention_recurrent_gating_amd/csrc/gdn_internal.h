// Internal interface between the C-ABI host code (gdn_api.cpp) and the
// device code (gdn_kernels.hip, gdn_rows.hip, gdn_chunk.hip).  Not installed;
// not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Everything one launch of the fused update needs.  Passed by value as the
// kernel argument.
struct FusedParams {
    const void* q;
    const void* k;
    const void* v;
    const void* a;
    const void* b;
    const float* g;             // precomputed log-decay [N, H_v] (unfused pair) or nullptr
    const float* beta;          // precomputed beta [N, H_v] (with g)
    const float* A_log;
    const float* dt_bias;
    void* pool;                 // state tiles, fp32 or bf16 (state_bf16)
    const int32_t* state_idx;
    const int32_t* cu_seqlens;  // nullptr: T tokens per sequence
    void* out;
    void* inter;                // nullptr: no intermediate states (same storage type)
    int64_t q_stride;           // elements between tokens
    int64_t k_stride;
    int64_t v_stride;
    int64_t ab_stride;          // elements between tokens of a and b
    int32_t ab_khead;           // elements between k-heads of a and b (dense: G)
    int32_t T;
    int32_t Hk;
    int32_t Hv;
    int32_t G;                  // Hv / Hk
    int32_t V;
    int32_t groups_per_khead;   // workgroups per (sequence, k-head)
    float scale;
    float eps;
    int32_t write_final;        // 0 under GDN_FLAG_NO_FINAL_WRITEBACK
    int32_t state_bf16;         // 1: pool and intermediates hold bf16
    int32_t state_vk;           // 1: tiles stored transposed (V x K); chunked kernel only
};

// Kernel families.
constexpr int kKindColumns = 0;  // wave = (v-head, BV-column tile); any token count
constexpr int kKindRows = 1;     // wave = (v-head, block of whole rows); any token count
constexpr int kKindValueRows = 2;  // transposed (VK) state: wave = (v-head, block of value-rows)
constexpr int kKindChunked = 3;    // workgroup = (sequence, v-head); 64-token chunks on MFMA

struct LaunchShape {
    int kind;
    int K;
    int block_v;      // columns per wavefront
    int block_k;      // rows per wavefront
    int act;          // 0 = fp32, 1 = bf16
    int multi_token;  // 0: one token per sequence; 1: token loop (kChunkTokens staged at a time)
    int waves;        // wavefronts per workgroup
    int rows_rpl_max; // row-split kernel: at most 32, 16 or 8 state rows per lane
    int chunk;        // tokens staged per chunk (1 for the single-token kernel)
    int64_t groups;   // grid size
    int lds_bytes;
};

// Tokens staged in LDS at a time by the per-token kernels' token loops.
constexpr int kChunkTokens = 16;

// Dynamic LDS bytes of a launch shape (V = head_v_dim).
int lds_bytes_for(const LaunchShape& shape, int V);

// True when a column-tile kernel instance exists for (K, block_v).
bool instance_exists(int K, int block_v);

// A fused-update kernel entry (every instance takes the parameter block by
// value).
using KernelFn = void (*)(FusedParams);

// The row-split kernel for (K, V, activation dtype, at most rpl_max rows per
// lane); multi_token selects the token-loop variant.  nullptr if none.
KernelFn select_rows(int K, int V, int act, int rpl_max, int multi_token);

// Rows per wavefront of the row-split kernel for (K, V) with at most rpl_max
// (32, 16 or 8) rows per lane; 0 if there is no such instance.
int rows_per_wave(int K, int V, int rpl_max);

// Value-rows per wavefront of the VK-layout kernel for (K, V); 0 if there is
// no instance for that pair.
int vk_rows_per_wave(int K, int V);

// Enqueues the standalone gating kernel (n = N*H_v outputs).
hipError_t launch_gating(const void* a, const void* b, const float* A_log, const float* dt_bias,
                         float* g, float* beta, int64_t n, int Hv, int G, int64_t ab_stride,
                         int32_t ab_khead, int act, hipStream_t stream);

// Static LDS bytes of the chunked kernel for (K, V, act); 0 if there is no
// instance (K, V in {32, 64, 128}).
int chunk_lds_bytes(int K, int V, int act);

// Value columns per wavefront of the chunked kernel (V / this = wavefronts).
int chunk_block_v();

// Tokens per chunk of the chunked kernel.
constexpr int kChunkedTokens = 64;

// Enqueues the chunked kernel (grid = sequences x v-heads).
hipError_t launch_chunked(const LaunchShape& shape, const FusedParams& p, hipStream_t stream);

// The two-kernel chunked form over a workspace: bytes of one (chunk slot,
// v-head) entry, the chunk slots of a call (entries = slots x H_v), and the
// launch of the prep kernel (slots x H_v workgroups) and the state pass
// (the chunked kernel's grid).
int64_t chunk_ws_entry_bytes();
int64_t chunk_ws_slots(int64_t num_tokens, int num_seqs);
hipError_t launch_chunked_ws(const LaunchShape& shape, const FusedParams& p, int num_seqs,
                             int64_t num_tokens, void* workspace, hipStream_t stream);

// The library's fixed device scratch (gdn_scratch.hip), the workspace of the
// allocation-free chunked entry point: its size, and its address on `device`
// (looked up with that device current on the first call for it).
size_t scratch_bytes();
hipError_t scratch_address(int device, void** out);

// Enqueues the fused kernel; returns the HIP launch status.
hipError_t launch_fused(const LaunchShape& shape, const FusedParams& p, hipStream_t stream);

}  // namespace gdn
