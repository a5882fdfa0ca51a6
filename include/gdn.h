/*
 * libgdn — fused sigmoid gating + gated delta-rule recurrent state update
 * (Gated DeltaNet decode) for AMD Instinct MI355X (gfx950).
 *
 * The operation is the fused kernel described by vLLM PR #35777
 * ("implementation" section: the gating that produced g and beta is folded
 * into the recurrent delta-rule update, which takes A_log, a, b and dt_bias
 * directly, normalises q/k with rsqrt, and has a speculative-decoding mode)
 * and tuned by sglang PR #18271 ("Benchmarking and Profiling": V-column
 * tiles, bs=512 on a TP4 shard).  Per token t, value head h and key head
 * j = h / G (G = H_v / H_k; consecutive v-heads share a k-head, as in the
 * per-k-head a/b grouping of vLLM PR #37975, implementation section):
 *
 *   g     = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h])
 *   beta  = sigmoid(b[t,h])
 *   khat  = k[t,j] * rsqrt(|k[t,j]|^2 + eps)
 *   qhat  = scale * q[t,j] * rsqrt(|q[t,j]|^2 + eps)      (scale default K^-1/2)
 *   S     = exp(g) * S
 *   u     = beta * (v[t,h] - S^T khat)
 *   S     = S + khat u^T
 *   out[t,h] = S^T qhat
 *
 * S is the K x V fp32 state of (sequence, v-head), gathered from and written
 * back to a slot-indexed pool, stored either with V fastest (GDN_LAYOUT_KV,
 * the default) or transposed with K fastest (GDN_LAYOUT_VK).  One call covers T=1 decode, fixed-T
 * multi-token verification and varlen sequences (cu_seqlens), with optional
 * per-token intermediate states.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers allocated by the caller; the
 *    library never allocates, frees or synchronises device memory (except
 *    GDN_FLAG_DEBUG_CHECKS, which copies the index arrays to the host).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns after the launch.
 *  - Errors are returned as gdn_status before anything is launched; a
 *    thread-local message (gdn_last_error_message) gives the detail.  No call
 *    aborts or throws.
 *  - The library keeps no state between calls and is re-entrant.  Calls that
 *    update the same pool slots must be ordered by the caller (same stream).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 2

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_NULL_POINTER = 1,      /* a required pointer is NULL              */
    GDN_ERR_BAD_SHAPE = 2,         /* negative/inconsistent sizes, H_v % H_k  */
    GDN_ERR_UNSUPPORTED_SHAPE = 3, /* K or V outside the supported set        */
    GDN_ERR_UNSUPPORTED_DTYPE = 4, /* act_dtype not F32/BF16                  */
    GDN_ERR_MISALIGNED = 5,        /* pointer or stride breaks the alignment  */
    GDN_ERR_LAUNCH = 6,            /* the HIP runtime rejected the launch     */
    GDN_ERR_BAD_ARGUMENT = 7,      /* other invalid argument (tile override,
                                      debug-check contract violation, ...)    */
} gdn_status;

typedef enum gdn_dtype {
    GDN_DTYPE_F32 = 0,
    GDN_DTYPE_BF16 = 1,
} gdn_dtype;

/* Leave the pool unchanged (spec verify whose acceptance is decided later:
 * the caller copies the accepted intermediate state itself). */
#define GDN_FLAG_NO_FINAL_WRITEBACK 0x1u
/* Before launching, copy state_idx (and cu_seqlens) to the host and check
 * the caller contract: non-negative slots distinct and < num_slots,
 * cu_seqlens[0] = 0, non-decreasing, cu_seqlens[B] = num_tokens.  Synchronous
 * on `stream`; meant for tests and debugging. */
#define GDN_FLAG_DEBUG_CHECKS 0x2u

/* Storage order of each K x V state tile in the pool and in
 * intermediate_states.  The layout is a property of the caller's buffers. */
#define GDN_LAYOUT_KV 0 /* element (kappa, c) at kappa*V + c (V fastest)      */
#define GDN_LAYOUT_VK 1 /* element (kappa, c) at c*K + kappa (K fastest): each
                           value-row is contiguous; served by the value-row
                           kernel, whose wavefronts never synchronise        */

typedef struct gdn_config {
    int32_t num_seqs;        /* B >= 0 sequences (B = 0, or num_tokens = 0:
                                nothing is launched, read or written, and the
                                activation pointers may be NULL)              */
    int32_t tokens_per_seq;  /* T >= 1 tokens per sequence when cu_seqlens is
                                NULL (sequence i owns token rows [i*T, i*T+T));
                                ignored with cu_seqlens                          */
    int64_t num_tokens;      /* N: rows of q, k, v, a, b, out, intermediate_states.
                                >= B*T without cu_seqlens; = cu_seqlens[B] with */
    int32_t num_k_heads;     /* H_k >= 1                                         */
    int32_t num_v_heads;     /* H_v >= 1, a multiple of H_k                      */
    int32_t head_k_dim;      /* K in {32, 64, 128, 256}                          */
    int32_t head_v_dim;      /* V in {32, 64, 128, 256}                          */
    int64_t num_slots;       /* rows of the state pool (bounds the slot indices) */
    int32_t act_dtype;       /* gdn_dtype of q, k, v, a, b and out               */
    float scale;             /* query scale; <= 0 selects K^-1/2                 */
    float l2norm_eps;        /* eps inside the rsqrt of the q/k norms (>= 0)     */
    int64_t q_stride_tok;    /* elements between consecutive tokens of q;
                                0 = dense (H_k*K).  Heads are dense within a token */
    int64_t k_stride_tok;    /* same for k                                       */
    int64_t v_stride_tok;    /* same for v (dense = H_v*V)                       */
    int64_t ab_stride_tok;   /* elements between tokens of a and b; 0 = dense H_v */
    int32_t ab_stride_khead; /* elements between the k-heads' groups of a and b;
                                0 = dense G.  Element (t, h) of a (and of b) is
                                read at t*ab_stride_tok + (h/G)*ab_stride_khead
                                + h%G, which reads a and b straight out of a
                                projection packed per k-head (vLLM PR #37975,
                                implementation: the a/b projection is reshaped
                                to (H_k, 2*H_v/H_k))                              */
    uint32_t flags;          /* GDN_FLAG_*                                       */
    int32_t state_layout;    /* GDN_LAYOUT_KV (0) or GDN_LAYOUT_VK (1)           */
    int32_t state_dtype;     /* storage of state_pool and intermediate_states:
                                GDN_DTYPE_F32 (0, default) or GDN_DTYPE_BF16.
                                The update runs in fp32 either way; bf16 tiles
                                are widened on load and rounded to nearest even
                                on store (half the state traffic)              */
    /* Tiling overrides (0 = the library's static table).  They change the
     * order of the fp32 reductions, never the operation. */
    int32_t kernel_family;   /* GDN_KERNEL_AUTO (0): the chunked kernel for
                                calls without intermediate states averaging at
                                least 32 tokens per sequence, or 16 when the
                                num_seqs * H_v workgroups fit one per CU
                                (256), both times sqrt(128*128 / (K*V))
                                (K, V <= 128);
                                otherwise, with GDN_LAYOUT_KV, row split
                                (column tiles where no row-split instance
                                fits, where block_v is set, and for token
                                loops without intermediate states at K, V <=
                                128 other than 128 x 128 from 1024
                                (sequence, k-head) workgroups, and for token
                                loops at 128 x 128 on fewer than 64); with
                                GDN_LAYOUT_VK,
                                value rows.  The host sees only the mean
                                length, so a batch with a few long sequences
                                among many short ones should ask for
                                GDN_KERNEL_CHUNKED itself: the per-token
                                kernels take one dependent step per token of
                                the longest sequence                           */
    int32_t block_v;         /* column tiles: 8, 16, 32 or 64 V-columns per
                                wavefront (dividing V).  A non-zero value with
                                GDN_KERNEL_AUTO selects the column tiles        */
    int32_t block_k;         /* row split: K-rows per wavefront (rows per lane
                                32, 16 or 8 times the rows one instruction
                                covers)                                        */
    int32_t waves_per_group; /* wavefronts per workgroup, 1..8: column tiles:
                                dividing G*V/block_v; row split: a multiple of
                                K/block_k covering a divisor of G heads        */
} gdn_config;

/* Kernel families (gdn_config.kernel_family, gdn_launch_info.kernel_family). */
#define GDN_KERNEL_AUTO 0
#define GDN_KERNEL_COLUMN_TILES 1 /* wavefront = (v-head, block_v columns, all K
                                     rows); any number of tokens               */
#define GDN_KERNEL_ROW_SPLIT 2    /* wavefront = (v-head, all V columns, block_k
                                     rows); any number of tokens               */
#define GDN_KERNEL_VALUE_ROWS 3   /* GDN_LAYOUT_VK only: wavefront = (v-head,
                                     block of whole value-rows); any number of
                                     tokens                                    */
#define GDN_KERNEL_CHUNKED 4      /* workgroup = (sequence, v-head): 64-token
                                     chunks in the WY form on the matrix cores
                                     (gdn_chunk_gated_delta_rule_fwd); either
                                     layout; K, V in {32, 64, 128}; writes no
                                     intermediate states; no tiling overrides  */

/* Describes the launch that a configuration maps to (gdn_plan). */
typedef struct gdn_launch_info {
    int32_t kernel_family;    /* the GDN_KERNEL_* family that runs           */
    int32_t block_v;          /* V-columns per wavefront                     */
    int32_t block_k;          /* K-rows per wavefront                        */
    int32_t waves_per_group;  /* wavefronts per workgroup                    */
    int32_t tokens_per_chunk; /* tokens staged in LDS at a time              */
    int32_t multi_token;      /* 0: single-token decode kernel; 1: token loop */
    int64_t workgroups;       /* grid size                                   */
    int32_t threads_per_group;
    int32_t lds_bytes;        /* LDS per workgroup                           */
} gdn_launch_info;

/* Fills `cfg` with defaults: scale 0 (K^-1/2), eps 1e-6, dense strides,
 * F32 activations, T = 1, library-chosen tiling. Sizes are zeroed. */
void gdn_default_config(gdn_config* cfg);

/*
 * The fused gating + gated delta-rule update (one launch).
 *
 *  q, k     [N, H_k, K]   act_dtype; token stride q/k_stride_tok elements
 *  v        [N, H_v, V]   act_dtype; token stride v_stride_tok
 *  a, b     [N, H_v]      act_dtype (dense, or strided per ab_stride_*)
 *  A_log, dt_bias [H_v]   fp32
 *  state_pool [num_slots, H_v, K, V] (GDN_LAYOUT_KV) or [num_slots, H_v,
 *             V, K] (GDN_LAYOUT_VK), fp32 or bf16 (state_dtype); updated in place
 *  state_idx  [B] int32: pool slot of sequence i; any negative value marks a
 *             padded sequence, which is skipped entirely (its pool rows, out
 *             rows and intermediate rows are neither read nor written)
 *  cu_seqlens [B+1] int32 token offsets, or NULL for T tokens per sequence.
 *             A zero-length sequence is skipped like a padded one.
 *  out      [N, H_v, V]   act_dtype, dense; bf16 is rounded to nearest even
 *  intermediate_states [N, H_v, K, V] fp32 (same tile layout as the pool) or
 *             NULL: row t receives S after
 *             token t (so the last token's row equals the final state)
 *
 * Alignment: q, k, v and out 16-byte aligned; state_pool and
 * intermediate_states 16-byte (fp32) or 8-byte (bf16) aligned; q/k/v token
 * strides multiples of 8 elements.
 * Caller contract (undefined if broken; checked under GDN_FLAG_DEBUG_CHECKS):
 * non-negative slot indices are distinct and < num_slots; cu_seqlens is
 * non-decreasing from 0 to N.  Rows of out/intermediate_states that belong to
 * no live token are not written.
 */
gdn_status gdn_gating_delta_rule_update(
    const void* q, const void* k, const void* v, const void* a, const void* b,
    const float* A_log, const float* dt_bias, void* state_pool,
    const int32_t* state_idx, const int32_t* cu_seqlens, void* out,
    void* intermediate_states, const gdn_config* cfg, void* stream);

/*
 * The unfused pair, for callers that keep the gates as tensors (vLLM PR
 * #35777 describes the fused op as replacing a separate gating kernel and a
 * recurrent update that consumes its g and beta).
 *
 * gdn_gating: g[t,h] = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h]) and
 * beta[t,h] = sigmoid(b[t,h]) for the cfg->num_tokens tokens (g, beta dense
 * fp32 [N, H_v]; a, b strided as in the fused call).  Uses num_tokens,
 * num_k_heads, num_v_heads, act_dtype and the ab strides of cfg.
 *
 * gdn_recurrent_update: the update of gdn_gating_delta_rule_update with
 * gamma = exp(g) and beta taken from those tensors.  The pair gives the
 * fused call's results bit for bit.
 */
gdn_status gdn_gating(const void* a, const void* b, const float* A_log, const float* dt_bias,
                      float* g, float* beta, const gdn_config* cfg, void* stream);

gdn_status gdn_recurrent_update(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, void* state_pool, const int32_t* state_idx,
                                const int32_t* cu_seqlens, void* out, void* intermediate_states,
                                const gdn_config* cfg, void* stream);

/*
 * The chunked forward (prefill) of the same operation: the results of
 * gdn_gating_delta_rule_update with intermediate_states = NULL (outputs and
 * final states, up to fp32 rounding), computed 64 tokens at a time in the WY
 * form of the chunked gated delta rule.  Meant for long sequences: the work
 * per chunk is dense matrix products, against one dependent step per token
 * in the per-token kernels.
 *
 * With a workspace (the fast form), two kernels run.  sglang PR #21411
 * (implementation section) builds a chunk's state-independent matrices --
 * the key Gram product and the triangular solve -- in a kernel of its own
 * over all chunks at once (chunk_gated_delta_rule_fwd, CHUNK_SIZE 64); here
 * too a first kernel builds, for every (chunk, v-head) in parallel, the full
 * inverse (I + L)^-1, the masked query-key products and the per-token
 * decays into `workspace`; a second kernel then walks each (sequence,
 * v-head)'s chunks in order with the state on chip, doing only the
 * state-dependent products.  workspace must be 256-byte aligned and hold at
 * least gdn_chunk_workspace_bytes(cfg) bytes (workspace_bytes says how many
 * it holds); it is caller-owned device scratch whose contents on entry do not
 * matter and on return are undefined.  Calls that run concurrently need
 * separate workspaces.
 *
 * With workspace = NULL (workspace_bytes ignored), one kernel does
 * everything: a workgroup per (sequence, v-head) builds each chunk's
 * matrices itself before its state products.  No scratch memory is used; it
 * is the form AUTO takes for long calls of gdn_gating_delta_rule_update.
 *
 * Arguments, layouts, alignment and the caller contract are otherwise those
 * of gdn_gating_delta_rule_update.  cfg->kernel_family must be
 * GDN_KERNEL_AUTO or GDN_KERNEL_CHUNKED, and block_v, block_k and
 * waves_per_group must be 0.  K and V must be 32, 64 or 128, and 64 token
 * rows of q, k, v, a, b or out must span less than 2 GiB.  A workspace that
 * is misaligned or too small is rejected (GDN_ERR_MISALIGNED,
 * GDN_ERR_BAD_ARGUMENT) before anything is launched.  gdn_recurrent_update
 * with kernel_family = GDN_KERNEL_CHUNKED runs the one-kernel form on
 * precomputed gates.
 */
gdn_status gdn_chunk_gated_delta_rule_fwd(
    const void* q, const void* k, const void* v, const void* a, const void* b,
    const float* A_log, const float* dt_bias, void* state_pool,
    const int32_t* state_idx, const int32_t* cu_seqlens, void* out,
    void* workspace, size_t workspace_bytes, const gdn_config* cfg, void* stream);

/* Bytes of workspace gdn_chunk_gated_delta_rule_fwd needs for `cfg`: one
 * 21,760-byte entry per (chunk slot, v-head), with floor(num_tokens / 64) +
 * num_seqs chunk slots (a sequence's chunks start at the slot after the
 * previous sequence's, rounded to 64-token boundaries).  0 when cfg is NULL
 * or describes no work (num_seqs or num_tokens 0), and for negative sizes. */
size_t gdn_chunk_workspace_bytes(const gdn_config* cfg);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * two-kernel form of gdn_chunk_gated_delta_rule_fwd over the library's own
 * fixed device scratch instead of a caller workspace.  Same arguments without
 * the workspace, same results bit for bit.
 *
 * The scratch is GDN_CHUNK_SCRATCH_BYTES (128 MiB) of device memory that each
 * GPU the library runs on holds until the process ends.  A call that needs
 * more (gdn_chunk_workspace_bytes(cfg) > GDN_CHUNK_SCRATCH_BYTES: (floor(N /
 * 64) + B) x H_v above 6168 chunk entries, e.g. about 11.8k tokens over 8
 * sequences at 32 v-heads) is rejected with GDN_ERR_BAD_ARGUMENT before
 * anything is launched.  Nothing in it needs clearing between calls.  Every
 * call on one GPU uses the same scratch: calls that may overlap on a GPU
 * (other streams, or host threads without ordering between them) race, and
 * the caller must serialise them.  The call allocates and frees nothing.
 */
#define GDN_CHUNK_SCRATCH_BYTES ((size_t)128 << 20)
gdn_status gdn_chunk_gated_delta_rule_fwd_noalloc(
    const void* q, const void* k, const void* v, const void* a, const void* b,
    const float* A_log, const float* dt_bias, void* state_pool,
    const int32_t* state_idx, const int32_t* cu_seqlens, void* out,
    const gdn_config* cfg, void* stream);

/* Host-side argument check of gdn_gating_delta_rule_update (same arguments,
 * no stream); launches nothing and never touches device memory. */
gdn_status gdn_validate(
    const void* q, const void* k, const void* v, const void* a, const void* b,
    const float* A_log, const float* dt_bias, const void* state_pool,
    const int32_t* state_idx, const int32_t* cu_seqlens, const void* out,
    const void* intermediate_states, const gdn_config* cfg);

/* The launch a valid configuration maps to (no device access), for a call
 * with or without cu_seqlens and intermediate_states. */
gdn_status gdn_plan(const gdn_config* cfg, int has_cu_seqlens, int has_intermediate_states,
                    gdn_launch_info* info);

/* Static description of a status code (never NULL).  Takes any int, so that
 * a value outside gdn_status (from another ABI version, say) is answered with
 * "unknown status" rather than read as an enumerator it is not. */
const char* gdn_status_string(int status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* gdn_last_error_message(void);

/* GDN_ABI_VERSION of the loaded library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
