/*
 * mlra.h -- C ABI of libmlra.so: decode-stage Multi-Head Low-Rank Attention
 * (MLRA) over a paged latent KV cache, on AMD Instinct MI355X (gfx950).
 *
 * What is computed (wispaper.ai blog "MLRA: Breaking the Sharding Bottleneck
 * in Latent Attention", section "The Core Insight: Sum of Branches, Not Sum
 * of Keys", and section "Mathematical Calibration: Scaling the Latents"):
 * the latent is split into n_branch branches; each branch b runs its own
 * softmax attention and the branch outputs are summed *after* attention and
 * multiplied by a fixed output factor. Keys are scored in absorbed form, so
 * the kernel only ever reads the cached latents c_b[t] and one decoupled RoPE
 * key k_r[t] per token that every branch shares (the blog's 1.5*dh per-rank
 * load: one dh-wide branch latent plus a 0.5*dh position key). For sequence s,
 * new query token j (0 <= j < Q), head h and branch b:
 *
 *   V      = L_s - (Q - 1 - j)   if causal, else L_s   (L_s = seq_lens[s])
 *   z[t]   = scale * (q_latent[s,j,h,b,:] . c_b[t] + q_rope[s,j,h,:] . k_r[t]),  t < V
 *   lse_b  = ln sum_{t<V} exp(z[t])
 *   o_b    = sum_{t<V} exp(z[t] - lse_b) * c_b[t]                 (latent space, DC wide)
 *   SUM    : out[s,j,h,:]   = out_rescale * sum_b o_b
 *   CONCAT : out[s,j,h,b,:] = out_rescale * o_b
 *   V <= 0 : o_b = 0 and lse_b = -inf.
 *
 * Token t of sequence s lives in physical block block_table[s][t / 64], slot
 * t % 64 of both caches. seq_lens counts the Q new tokens, which must already
 * be in the cache.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing and keeps no state besides cached device properties.
 *  - Calls are asynchronous: they enqueue work on `stream` (a hipStream_t;
 *    NULL = the default stream) and return. Buffers must stay alive until the
 *    stream reaches that point.
 *  - Host-side validation is synchronous, reads no device memory, and on
 *    failure returns a status without enqueuing anything. MLRA_ERR_HIP means a
 *    launch failed (hipGetLastError); the stream may hold partial work.
 *  - No exceptions cross the ABI and the library prints nothing.
 *  - Two calls that share a workspace must not run concurrently.
 *  - Every workspace (decode, prefill, output projection) starts with a
 *    header of MLRA_DECODE_WS_HEADER_BYTES that belongs to decode calls and
 *    that the other calls leave untouched, so one scratch buffer can serve
 *    them all. It must hold zeros before the buffer's first decode call
 *    (allocate it zero-filled, or call mlra_decode_workspace_init once);
 *    every call leaves it ready for the next one. The rest of a workspace
 *    needs no initialisation. The header holds a status word
 *    (mlra_decode_read_status) and the counters through which the split
 *    kernel's workgroups merge their results without a second launch.
 */
#ifndef MLRA_H_
#define MLRA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mlra_status {
  MLRA_OK = 0,
  MLRA_ERR_NULL_PTR = 1,     /* a required pointer is NULL */
  MLRA_ERR_BAD_DIMS = 2,     /* a size is out of range or inconsistent */
  MLRA_ERR_UNSUPPORTED = 3,  /* valid, but no kernel is built for this shape */
  MLRA_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than required */
  MLRA_ERR_ALIGNMENT = 5,    /* pointer or stride breaks the 16-byte rule */
  MLRA_ERR_HIP = 6           /* a HIP runtime call or launch failed */
} mlra_status;

typedef enum mlra_dtype {
  MLRA_BF16 = 0,  /* q, caches and out in bfloat16; MFMA path */
  MLRA_FP32 = 1   /* q, caches and out in float32; vector-ALU path */
} mlra_dtype;

typedef enum mlra_branch_reduce {
  MLRA_BRANCH_SUM = 0,    /* out[S][Q][H][DC] = out_rescale * sum_b o_b */
  MLRA_BRANCH_CONCAT = 1  /* out[S][Q][H][n_branch][DC] = out_rescale * o_b */
} mlra_branch_reduce;

/* Bytes at the start of every decode workspace that hold the status word and
 * the in-kernel merge counters (zero before first use; see above). The
 * per-split partial results follow at this offset. */
#define MLRA_DECODE_WS_HEADER_BYTES 65792

/* mlra_decode_dims.flags */
#define MLRA_DECODE_FLAG_FUSED_MERGE 1  /* let the split kernel merge the splits itself where
                                           it can (see mlra_decode_attention) */

/* Status bits (mlra_decode_read_status). */
#define MLRA_DEVSTATUS_WAIT_EXPIRED 1u  /* a bounded wait inside the split kernel gave up:
                                           that call's out and lse are unreliable */
#define MLRA_DEVSTATUS_MERGE_FAILED 2u  /* the in-kernel merge could not verify that a
                                           sequence's workgroups shared one L2 (XCD), or
                                           its waits expired: that sequence's out and lse
                                           were written as NaN */

/* Shapes and layout of one decode call. Strides are in ELEMENTS; 0 selects the
 * dense default. The innermost (feature) dimension is always contiguous. */
typedef struct mlra_decode_dims {
  int32_t num_seqs;            /* S  >= 1 */
  int32_t q_len;               /* Q  in {1, 2, 3, 4}: new query tokens per sequence
                                * (decode; longer chunks go to mlra_prefill_attention,
                                * which computes the same out and lse for any Q) */
  int32_t num_heads;           /* H  >= 1, H * Q <= 128 (decode) */
  int32_t d_latent;            /* DC per branch: fp32 {64, 128, 256, 512}; bf16 {64, 128} with
                                  any n_branch, 256 with n_branch <= 2 and DR = 64 (MLRA-2:
                                  MLA's 512-wide latent in two branches), 512 with n_branch = 1
                                  and DR = 64 (MLA); other bf16 shapes: MLRA_ERR_UNSUPPORTED */
  int32_t d_rope;              /* DR in {32, 64} */
  int32_t block_size;          /* tokens per cache block; must be 64 */
  int32_t max_blocks_per_seq;  /* columns of block_table */
  int32_t num_blocks;          /* physical blocks in each cache */
  int32_t max_seq_len;         /* host-side upper bound of seq_lens (no device read needed) */
  int32_t causal;              /* nonzero: query j sees t < L - (Q - 1 - j) */
  int32_t num_splits;          /* 0: library plans split-K; >0: at most this many splits per
                                * sequence, raised where a split would exceed 1024 tiles
                                * (65536 tokens) for bfloat16 */
  int32_t dtype;               /* mlra_dtype */
  int32_t reduce;              /* mlra_branch_reduce */
  int32_t flags;               /* MLRA_DECODE_FLAG_* bits (0 = defaults); others must be 0 */
  /* latent_cache element strides: block, token, branch. Defaults (0):
   * token-major [num_blocks][64][n_branch][DC] -> 64*n_branch*DC, n_branch*DC, DC */
  int64_t latent_stride_block, latent_stride_token, latent_stride_branch;
  /* rope_cache element strides: block, token. Defaults: [num_blocks][64][DR] */
  int64_t rope_stride_block, rope_stride_token;
  /* Optional host-side sum of seq_lens (0 = unknown: plan as if every
   * sequence had max_seq_len). Only steers how tokens are split across
   * workgroups (decode) and whether workgroups are ordered by their work
   * (prefill); results do not depend on it. */
  int64_t sum_seq_lens;
} mlra_decode_dims;

/* Split-K plan, computed on the host from dims alone (no device read). On
 * the device each sequence uses ceil(ceil(L/64) / tiles_per_split) of its
 * splits_per_seq splits (row_groups workgroups each); the rest exit at once. */
typedef struct mlra_decode_plan {
  int32_t num_cus;             /* compute units the plan targets */
  int32_t target_groups;       /* split-kernel workgroups the planner aims for */
  int32_t waves_per_group;     /* waves in one split-kernel workgroup */
  int32_t tiles_per_split;     /* 64-token tiles one workgroup (one split) covers */
  int32_t splits_per_seq;      /* splits of the longest sequence; grid = S x this */
  int32_t kernel_variant;      /* internal kernel id (for logs and tests) */
  int32_t lds_bytes;           /* LDS one split workgroup allocates */
  int32_t row_groups;          /* split-kernel workgroups per split (1 to 4): branch
                                  groups times row groups, when the call's branches and
                                  32-row tiles of query rows do not fit one workgroup */
  int32_t fused_merge;         /* 1: the split kernel merges the splits itself, with no
                                  combine launch (see mlra_decode_attention) */
  int32_t reserved0;
  size_t workspace_bytes;      /* bytes of device workspace the call needs (header included) */
} mlra_decode_plan;

/* Plan a call without touching the GPU: split sequences into chunks of
 * tiles_per_split 64-token tiles so that about target_groups workgroups run.
 * num_cus <= 0 queries the current device (needs HIP); pass e.g. 256 to plan
 * for an MI355X on a host without a GPU. Returns the same validation errors
 * as mlra_decode_attention, minus the pointer checks. */
mlra_status mlra_decode_make_plan(const mlra_decode_dims* dims, int32_t n_branch,
                                  int32_t num_cus, mlra_decode_plan* plan);

/* Workspace bytes for a call on the current device (queries its CU count). */
mlra_status mlra_decode_workspace_size(const mlra_decode_dims* dims, int32_t n_branch,
                                       size_t* bytes);

/* Zero the header of a decode workspace (asynchronous on stream, by a small
 * kernel, so it may be captured into a HIP graph). Needed once per workspace
 * unless it was allocated zero-filled. bytes >= MLRA_DECODE_WS_HEADER_BYTES. */
mlra_status mlra_decode_workspace_init(void* workspace, size_t bytes, void* stream);

/* Read the status word of a decode workspace: MLRA_DEVSTATUS_* bits that
 * calls on it have set since it was last cleared (0: nothing went wrong).
 * Synchronous: waits for stream to reach this point, so not for graph
 * capture. clear != 0 then zeroes the word. */
mlra_status mlra_decode_read_status(void* workspace, uint32_t* bits, int32_t clear,
                                    void* stream);

/*
 * MLRA decode attention (formula above).
 *
 *  q_latent     [S][Q][H][n_branch][DC]   dtype, dense
 *  q_rope       [S][Q][H][DR]             dtype, dense; shared by all branches
 *  latent_cache paged, see latent_stride_*; dtype
 *  rope_cache   paged, see rope_stride_*;   dtype
 *  block_table  [S][max_blocks_per_seq]   int32, physical block ids in [0, num_blocks)
 *  seq_lens     [S]                       int32, device; 0 <= L <= max_seq_len
 *  n_branch     branches in the cache and in q_latent: {1, 2, 4}
 *  scale        softmax scale on the raw dot products (finite, > 0)
 *  out_rescale  output factor (finite); 1/sqrt(4) for MLRA-4
 *  out          SUM: [S][Q][H][DC]; CONCAT: [S][Q][H][n_branch][DC]; dtype
 *  lse          [S][Q][H][n_branch] float32, natural log; -inf where V <= 0
 *  workspace    device scratch of at least mlra_decode_workspace_size bytes,
 *               16-byte aligned; its first MLRA_DECODE_WS_HEADER_BYTES must be
 *               zero before its first decode call (see the conventions above)
 *
 * By default a second kernel merges the splits. With
 * MLRA_DECODE_FLAG_FUSED_MERGE, when the plan reports fused_merge (bfloat16;
 * S a multiple of 8 and at most 64; one workgroup per CU covers the whole
 * call; every sequence the same length bound), the split kernel finishes the
 * call itself: all workgroups of a sequence run on one XCD,
 * each publishes its partial result through that XCD's shared L2 and a
 * per-workgroup counter in the header, waits for the others and merges a
 * slice of the sequence's output. The workgroups verify that they share an
 * XCD; if they cannot (or their bounded waits expire), a workgroup that was
 * dispatched after all others of its sequence merges what the rest gave up,
 * or the sequence's out and lse are written as NaN and the status word says
 * so. On an MI355X this measured slower than the second kernel at B=16,
 * T=8192 (21.4 against 19.0 us per call): under load every round trip
 * through the L2 costs about 1 us, and the merge needs several.
 *
 * Alignment: every tensor pointer 16-byte aligned; cache strides multiples
 * of 16 bytes. Table entries past ceil(L/64) are never used (they may hold
 * anything; the kernel may load but never dereferences them). Cache rows
 * past L inside a sequence's last block may be loaded but never enter the
 * arithmetic (they may hold NaN). Memory safety on bad input: a seq_lens
 * entry above max_seq_len is treated as max_seq_len, and a table entry
 * outside [0, num_blocks) reads block 0 instead; both give wrong results
 * for that sequence but never an out-of-bounds access. Results are
 * deterministic: repeated calls with the same inputs, dims and device give
 * bit-identical out and lse.
 */
mlra_status mlra_decode_attention(const void* q_latent, const void* q_rope,
                                  const void* latent_cache, const void* rope_cache,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  int32_t n_branch, float scale, float out_rescale,
                                  void* out, float* lse, const mlra_decode_dims* dims,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * mlra_decode_attention with the library's own device scratch in place of a
 * workspace. Same arguments, results and errors as mlra_decode_attention,
 * minus workspace and workspace_bytes. The scratch is a fixed array of
 * MLRA_STATIC_SCRATCH_BYTES in the library's code object: every GPU that
 * loads the library holds one, zero-filled, until the process ends; the
 * call allocates nothing and frees nothing. A call whose plan needs more
 * (mlra_decode_make_plan's workspace_bytes) returns MLRA_ERR_WORKSPACE
 * before enqueuing anything. All calls on one GPU share its scratch, which
 * keeps the last call's contents (the header is left ready for the next
 * call): calls that overlap on one GPU (other streams, other host threads)
 * race and must not be issued.
 */
#define MLRA_STATIC_SCRATCH_BYTES (64u << 20)

mlra_status mlra_decode_attention_static(const void* q_latent, const void* q_rope,
                                         const void* latent_cache, const void* rope_cache,
                                         const int32_t* block_table, const int32_t* seq_lens,
                                         int32_t n_branch, float scale, float out_rescale,
                                         void* out, float* lse, const mlra_decode_dims* dims,
                                         void* stream);

/*
 * MLA-shaped comparison call: a single latent head (n_branch = 1, typically
 * DC = 512 plus DR = 64, the 4.5*dh per-token load the blog attributes to MLA),
 * one softmax, out_rescale = 1. Same argument rules as mlra_decode_attention;
 * out is [S][Q][H][DC] and lse [S][Q][H].
 */
mlra_status mla_decode_attention(const void* q_latent, const void* q_rope,
                                 const void* latent_cache, const void* rope_cache,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 float scale, void* out, float* lse,
                                 const mlra_decode_dims* dims, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * The two halves of mlra_decode_attention, for callers that schedule or time
 * them separately, or that merge partial results of one sequence computed
 * elsewhere (e.g. a context range held by another device) before combining.
 * Split-K with a log-sum-exp merge is exact: every split's softmax is
 * normalised on its own and re-weighted by exp(lse_split - lse_total).
 *
 * mlra_decode_partials runs the split kernel only (never the fused merge).
 * It takes the arguments of mlra_decode_attention that the scores need and
 * leaves, in the workspace, with P = plan.splits_per_seq, T =
 * plan.tiles_per_split, R = Q*H, row r = j*H + h (plan from
 * mlra_decode_make_plan with the same dims on the same device) and
 * H0 = MLRA_DECODE_WS_HEADER_BYTES:
 *   part_o   float32 [S][P][n_branch][R][DC] at byte offset H0:
 *            split k's softmax-weighted latent output over its tokens
 *            (already divided by its own sum of weights; 0 if it saw none);
 *   part_lse float32 [S][P][n_branch][R] at byte offset
 *            H0 + round_up(S*P*n_branch*R*DC*4, 256): natural log of the
 *            split's sum of exp(scaled score), -inf if it saw no visible token.
 * Split k of sequence s covers tokens [64*T*k, min(64*T*(k+1), L)); only the
 * splits k < ceil(ceil(L/64) / T) are written, the rest of the slots keep
 * whatever they held.
 *
 * mlra_decode_combine runs the combine kernel only: it merges the splits of
 * each (sequence, row, branch), applies the branch reduction and out_rescale,
 * and writes out and lse exactly as mlra_decode_attention does. It must get
 * the dims, n_branch and seq_lens of the partials call it follows, on the
 * same device and the same stream (or after it). Errors as for
 * mlra_decode_attention, checking only the pointers each half uses.
 */
mlra_status mlra_decode_partials(const void* q_latent, const void* q_rope,
                                 const void* latent_cache, const void* rope_cache,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 int32_t n_branch, float scale, const mlra_decode_dims* dims,
                                 void* workspace, size_t workspace_bytes, void* stream);

mlra_status mlra_decode_combine(const int32_t* seq_lens, int32_t n_branch, float out_rescale,
                                void* out, float* lse, const mlra_decode_dims* dims,
                                const void* workspace, size_t workspace_bytes, void* stream);

/*
 * Append the Q new tokens of every sequence to the paged caches: the step
 * before decode attention. What a token holds follows the wispaper.ai blog
 * "MLRA: Breaking the Sharding Bottleneck in Latent Attention", "The Core
 * Insight" (one latent per branch plus one decoupled position key shared by
 * the branches) and "Mathematical Calibration" (the latents are multiplied by
 * a calibration factor, here a caller argument).
 *
 *  latent_new   [S][Q][n_branch][DC] float32, dense: the new tokens' projected
 *               branch latents
 *  rope_new     [S][Q][DR] float32, dense: their projected position keys, not
 *               yet rotated
 *  latent_cache, rope_cache, block_table, seq_lens, n_branch, dims: as for
 *               mlra_decode_attention (same dims; num_heads, max_seq_len,
 *               causal, num_splits, reduce and sum_seq_lens are validated
 *               but not used here)
 *  latent_scale calibration factor on the latents (finite)
 *  rope_base    rotary base (finite, > 0; 10000 is the usual value)
 *
 * seq_lens counts the new tokens, so token j of sequence s lands at position
 * p = seq_lens[s] - Q + j: block block_table[s][p / 64], slot p % 64.
 *   latent row b   = latent_scale * latent_new[s][j][b]
 *   key pair i     = rotary embedding: (k[2i], k[2i+1]) turned by
 *                    the angle p * rope_base^(-2i/DR)
 * Each value is formed in double and rounded once to the cache dtype
 * (bf16: nearest, ties to even). Tokens whose position is negative or lies
 * past max_blocks_per_seq * 64, or whose block id is outside
 * [0, num_blocks), are not written. Asynchronous on stream; alignment as for
 * mlra_decode_attention (inputs and caches 16-byte aligned).
 */
mlra_status mlra_cache_append(const float* latent_new, const float* rope_new,
                              void* latent_cache, void* rope_cache,
                              const int32_t* block_table, const int32_t* seq_lens,
                              int32_t n_branch, float latent_scale, float rope_base,
                              const mlra_decode_dims* dims, void* stream);

/*
 * The output side of decode as one contraction, in bf16 with float32
 * accumulation:  y[M][D] = x[M][K] . W^T.
 * Following the wispaper.ai blog "MLRA: Breaking the Sharding Bottleneck in
 * Latent Attention", "The Core Insight" (branch outputs are combined after
 * attention), with one value up-projection W_UV[h][b] (dv x DC) per branch
 * and the output projection W_O (D x H*dv):
 *  x  [M][K] bf16, dense: the CONCAT output of mlra_decode_attention viewed
 *     as [S*Q][H*n_branch*DC] (M = S*Q, K = H*n_branch*DC; it already carries
 *     out_rescale)
 *  W  [D][K] bf16: the absorbed weight
 *     W[n][(h*n_branch + b)*DC + c] = sum_d W_O[n][h*dv + d] * W_UV[h][b][d][c]
 *  y  [M][D] bf16, dense (nearest, ties to even)
 * W is a fixed weight: mlra_out_projection_pack rewrites it once, on the
 * stream, into the order the kernel loads (D*K*2 bytes, caller-owned):
 *     packed[g][kb][w][q][l][e] = W[128g + 16w + l%16][64kb + 32q + 8(l/16) + e]
 * for g < D/128, kb < K/64, w < 8, q < 2, l < 64, e < 8; mlra_out_projection takes
 * the packed weight. Sizes: 1 <= M <= 128 (decode rows; larger M is an
 * ordinary GEMM), K a multiple of 512, D a multiple of 128; otherwise
 * MLRA_ERR_UNSUPPORTED. workspace: at least
 * mlra_out_projection_workspace_size bytes (0 for some sizes, then it may be
 * NULL), 16-byte aligned, no initialisation needed. Pointers 16-byte
 * aligned. Both calls are asynchronous on stream.
 */
mlra_status mlra_out_projection_pack(const void* w, void* w_packed, int32_t k, int32_t d,
                                     void* stream);

mlra_status mlra_out_projection_workspace_size(int32_t m, int32_t k, int32_t d, size_t* bytes);

mlra_status mlra_out_projection(const void* x, const void* w_packed, void* y, int32_t m,
                                int32_t k, int32_t d, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * Chunked-prefill MLRA attention: the decode formula at the top of this
 * header for a chunk of many new query tokens per sequence (many queries
 * per key, so the work is bound by matrix throughput rather than by HBM),
 * over the same paged latent cache
 * (wispaper.ai blog "MLRA: Breaking the Sharding Bottleneck in Latent
 * Attention", "The Core Insight": every head scores the shared latent and
 * RoPE key of each token, one softmax per branch, branch outputs combined
 * after attention). Token j of the chunk sits at position L - Q + j; with
 * causal set it sees every token up to its own position,
 * t < L - (Q - 1 - j). The chunk's latents and keys must already be in the
 * cache (mlra_cache_append), so a whole-sequence prefill is Q = L.
 *
 * Arguments, layouts, outputs, alignment and error rules as for
 * mlra_decode_attention, except:
 *  - q_len may be any value >= 1 (num_heads * q_len <= 2^26);
 *  - bf16 only, d_latent in {64, 128}, d_rope in {32, 64}, n_branch in
 *    {1, 2, 4}; other shapes (and fp32) give MLRA_ERR_UNSUPPORTED;
 *  - num_splits: 0 lets the library split long contexts when the query rows
 *    alone do not fill the GPU; > 0 asks for that many token splits; either
 *    way a split covers at most 1024 64-token tiles (65536 tokens) and longer
 *    contexts get more splits;
 *  - the workspace is needed only with more than one split, or with
 *    MLRA_BRANCH_SUM over more than one branch: mlra_prefill_workspace_size
 *    returns 0 otherwise, and workspace may then be NULL;
 *  - shapes whose grid would pass 2^31 - 1 workgroups (attention, or the
 *    merge of splits and branches) give MLRA_ERR_UNSUPPORTED.
 * When the lengths may differ (sum_seq_lens 0, or below num_seqs *
 * max_seq_len) and the call has at most 1024 (sequence, row group, split)
 * items, workgroups take them longest first, ranked on the device from
 * seq_lens. Results are deterministic: repeated calls give bit-identical out
 * and lse, whatever the order. mlra_prefill_make_plan fills the decode plan struct: row_groups counts
 * 256-row workgroups per sequence and branch, kernel_variant is 8.
 */
mlra_status mlra_prefill_make_plan(const mlra_decode_dims* dims, int32_t n_branch,
                                   int32_t num_cus, mlra_decode_plan* plan);

mlra_status mlra_prefill_workspace_size(const mlra_decode_dims* dims, int32_t n_branch,
                                        size_t* bytes);

mlra_status mlra_prefill_attention(const void* q_latent, const void* q_rope,
                                   const void* latent_cache, const void* rope_cache,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   int32_t n_branch, float scale, float out_rescale,
                                   void* out, float* lse, const mlra_decode_dims* dims,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Measurement helper, not part of the attention path: read `bytes` bytes
 * from src with `workgroups` workgroups of 512 threads (each a contiguous
 * chunk of bytes / workgroups, 16 bytes per lane per load, 8 loads per lane
 * in flight), folding them so that no load is dropped; sink[workgroups]
 * (uint32) is written only for one data pattern in 2^32. bench.py times it
 * in the same run as the decode kernels, at their launch shape, as the
 * streaming-read ceiling they are compared with. bytes must be a multiple
 * of 16 * workgroups; src 16-byte aligned. Asynchronous on stream.
 */
mlra_status mlra_stream_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink,
                             void* stream);

/* Static, never-NULL description of a status code. */
const char* mlra_status_string(mlra_status status);

/* Testing only: bound every later decode call's internal waits by `polls`
 * LDS polls and `polls` ticks (10 ns) of the in-kernel merge, so that tests
 * can make them expire and check the status path while every kernel still
 * ends; polls < 0 restores the defaults. Process-wide; not for production. */
mlra_status mlra_testing_set_wait_limit(int32_t polls);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t mlra_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLRA_H_ */
