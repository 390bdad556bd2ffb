/*
 * mla_dcp.h -- C ABI of the sequence-sharded MLA decode library (gfx950).
 *
 * One decode step of multi-head latent attention (MLA): H query heads share
 * one latent KV head whose per-token row holds 512 latent and 64 rope
 * dimensions ("GLM-5.2 vLLM Decode Context Parallelism", section "Understand
 * the cache-copy opportunity"; "The Final Verification: Confirming a 200k
 * Context Deployment on GLM-5", section "The Decision-Making Process Visible
 * in the Reasoning").  The cache is sharded along the sequence: global token
 * p of a request lives on shard p mod N as that shard's local token p div N
 * ("How vLLM Serves GLM-5.3 with Million-Token Contexts on 16 H200s", section
 * "The core design").  Each shard returns a partial output and the softmax
 * log-sum-exp of its tokens; the LSE merge combines the partials into the
 * full-context result ("GLM-5.2 vLLM Decode Context Parallelism", section
 * "See why vLLM 0.26.0 fails").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor arguments are DEVICE pointers unless stated otherwise.  The caller
 *   owns all memory; the library keeps no pointer after a call returns and
 *   allocates no device memory inside any call.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *   is enqueued asynchronously on it; inputs must stay valid and outputs
 *   untouched until it completes.
 * - Every call validates its arguments on the host and returns a status
 *   before anything is enqueued.  On a non-zero status nothing is enqueued
 *   and no output is written.
 * - Inputs and outputs must not alias.  Pointers to q, the KV pool and all
 *   outputs must be 16-byte aligned (MLA_ERR_ALIGN otherwise).
 * - Empty rows are never undefined: a (request, query token) with no token to
 *   attend on a shard yields output 0 and LSE -inf ("GLM-5.2 vLLM Decode
 *   Context Parallelism", section "Separate the backend merge from stable").
 *
 * Layouts (row-major, innermost last)
 * -----------------------------------
 *   q            [B][Tq][H][576]        q_dtype; 512 latent then 64 rope dims
 *   kv_pool      [pool_blocks][64][row] one row per token:
 *                  MLA_F32    576 x f32                          (2304 B)
 *                  MLA_BF16   576 x bf16                         (1152 B)
 *                  MLA_FP8_DS 512 x E4M3FN code, 4 x f32 scale (one per
 *                             128-dim group), 64 x bf16 rope     ( 656 B)
 *                  latent value d = decode(code[d]) * scale[d / 128]
 *   block_table  [B][max_blocks] int32, ONE shard's table: local token j of
 *                request b is row (j % 64) of pool block block_table[b][j/64]
 *   context_lens [B] int32: tokens in request b's whole (unsharded) cache,
 *                including the Tq query tokens' own rows; query token t
 *                (0 <= t < Tq) sits at global position L_b - Tq + t and
 *                attends positions 0 .. L_b - Tq + t
 *   topk_idx     [B][Tq][topk] int32 GLOBAL positions (negative = unused);
 *                a shard attends only the entries it owns (sparse mode).
 *                The list is a multiset: every non-negative entry is one
 *                term of the softmax, so a position listed twice is attended
 *                twice (weight 2 exp(s) in the normaliser and in the output)
 *   o_partial    [B*Tq][H][512] out_dtype     (token/head form)
 *   lse          [B*Tq][H] f32, natural log of sum exp(scale * q.k)
 *
 * Device-detected errors
 * ----------------------
 * A block-table row too narrow for a request's local length, a block id
 * outside [0, pool_blocks), or a top-K index outside the query token's causal
 * prefix sets a bit in the first 32-bit word of the workspace; the offending
 * tokens are skipped (treated as not attended).  The cache-write calls report
 * their own bad entries the same way (the write is skipped).  The word is sticky: it is
 * cleared only by mla_clear_device_error, and read by mla_get_device_error.
 */
#ifndef MLA_DCP_H
#define MLA_DCP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MLA_OK 0
#define MLA_ERR_NULL 1        /* a required pointer is NULL                    */
#define MLA_ERR_SHAPE 2       /* a size is out of range or inconsistent        */
#define MLA_ERR_SHARD 3       /* shard id / shard range / shard count invalid  */
#define MLA_ERR_UNSUPPORTED 4 /* head count, dimension or dtype not built      */
#define MLA_ERR_WORKSPACE 5   /* workspace smaller than the size query         */
#define MLA_ERR_DEVICE 6      /* a HIP runtime call failed                     */
#define MLA_ERR_ALIGN 7       /* a pointer is not 16-byte aligned              */

/* Element / row formats. */
#define MLA_F32 0
#define MLA_BF16 1
#define MLA_FP8_DS 2

/* Bits of the device error word. */
#define MLA_DEVERR_BLOCK_TABLE 1u /* table too narrow, or block id out of pool */
#define MLA_DEVERR_INDEX 2u       /* top-K index beyond the causal prefix      */
#define MLA_DEVERR_SLOT 4u        /* cache-write slot at or past the pool end  */
#define MLA_DEVERR_SCORES 8u      /* score row shorter than the visible prefix */
#define MLA_DEVERR_QUERY 16u      /* varlen query offsets not a partition      */

/* Shape of one decode step.  Fixed by this build: kv_lora_rank = 512,
 * rope_dim = 64, block_size = 64; num_heads in {16, 32, 64, 128} (the query
 * head envelope, "GLM-5.2 vLLM Decode Context Parallelism", section
 * "Calculate the GLM-5.2 head envelope": heads are padded to a supported
 * envelope and anything else is refused, not run). */
typedef struct mla_decode_desc {
    int32_t batch;        /* B >= 0 (0 = nothing to do)                    */
    int32_t q_len;        /* Tq >= 1 query tokens per request               */
    int32_t num_heads;    /* H                                              */
    int32_t kv_lora_rank; /* must be 512                                    */
    int32_t rope_dim;     /* must be 64                                     */
    int32_t block_size;   /* must be 64                                     */
    int32_t max_blocks;   /* width of each block-table row, >= 1            */
    int32_t topk;         /* 0 = dense; else entries per query token (<= 65536) */
    int32_t q_dtype;      /* MLA_F32 (with MLA_F32 cache) or MLA_BF16       */
    int32_t kv_dtype;     /* MLA_F32, MLA_BF16 or MLA_FP8_DS                */
    int32_t out_dtype;    /* MLA_F32 or MLA_BF16                            */
    float softmax_scale;  /* finite and > 0; scores are scale * q.k         */
    int64_t pool_blocks;  /* number of blocks in kv_pool, >= 1              */
} mla_decode_desc;

/* Human-readable name of a status code (static string, never NULL). */
const char* mla_status_string(int32_t status);

/* Tokens of a context of length context_len that shard shard_id of n_shards
 * stores under round-robin ownership: ceil((L - s) / N) for s < L, else 0.
 * Returns -1 for invalid arguments (n_shards < 1, shard outside [0, N),
 * negative length).  Host function. */
int32_t mla_shard_local_len(int32_t context_len, int32_t shard_id, int32_t n_shards);

/* Bytes of one cache row for a kv dtype (2304, 1152, 656), or -1. */
int64_t mla_kv_row_bytes(int32_t kv_dtype);

/* Workspace bytes that mla_decode_partial (shard_count = 1) or
 * mla_decode_partial_shards (shard_count shards) needs for `desc`.  Pure host
 * function: validates desc (same checks and codes as the decode calls) and
 * writes the size to *bytes_out.  The size is at least 256 (the device error
 * word lives in the first 4 bytes).  Beyond the error word the workspace
 * holds the step's transient state: the chunk plan and the float32 partial
 * outputs of rows split into chunks (their combine is the LSE merge below),
 * and, for a top-K step over a bf16 cache, each (shard, query token) row's
 * list of the pool rows it owns (int32, the top-K width rounded up to 32),
 * bounded by desc alone, so a caller can reserve it once, apart from the
 * cache pool.  Keeping the attention workspace a known, separately measured
 * allocation is what "GLM-5.2 vLLM Decode Context Parallelism", section
 * "Measure capacity and service behavior" asks for after a decode OOM inside
 * the attention kernel's own workspace. */
int32_t mla_decode_workspace_size(const mla_decode_desc* desc, int32_t shard_count,
                                  int64_t* bytes_out);

/* Partial decode attention of ONE shard (the call one DCP rank makes).
 * Computes, for every request b, query token t and head h, attention over the
 * tokens shard `shard_id` of `n_shards` owns (dense: all owned positions in
 * the causal prefix; sparse: owned entries of topk_idx[b][t]), writing the
 * normalised partial output and its LSE ("GLM-5.2 vLLM Decode Context
 * Parallelism", sections "See why vLLM 0.26.0 fails" and "Separate the backend
 * merge from stable").  1 <= n_shards <= 4096 and 0 <= shard_id < n_shards
 * (else MLA_ERR_SHARD).  topk_idx must be NULL when desc->topk == 0 and
 * non-NULL otherwise.  workspace: device memory of workspace_bytes >=
 * mla_decode_workspace_size(desc, 1); its first word is the sticky device
 * error word, the rest is scratch overwritten by the call. */
int32_t mla_decode_partial(const mla_decode_desc* desc, const void* q, const void* kv_pool,
                           const int32_t* block_table, const int32_t* context_lens,
                           const int32_t* topk_idx, int32_t shard_id, int32_t n_shards,
                           void* o_partial, float* lse, void* workspace,
                           int64_t workspace_bytes, void* stream);

/* mla_decode_partial for callers that cannot allocate or pass a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * device allocation.  Instead of a workspace the call uses a scratch array
 * the library holds on each GPU (64 MiB, allocated with the library's code
 * object on that device and kept until the process ends; its address is
 * looked up once per device).  Nothing is allocated inside the call.
 * Same inputs, outputs, checks and results as mla_decode_partial, except:
 *   err_word   device pointer to a 32-bit word that receives the device
 *              error bits (ORed in, never cleared by the call; read it with
 *              mla_get_device_error(err_word, ...)), or NULL to drop them
 * A call whose chunk plan and partials would not fit in the scratch plans
 * fewer, longer chunks; if even that does not fit it returns
 * MLA_ERR_WORKSPACE (a call of more than about a million query tokens).  A
 * top-K step over a bf16 cache whose per-row lists would not fit (more than
 * about 16 million list entries) runs on the slower vector kernel instead
 * (results within the same bounds against the definition, not bit for bit
 * those of the workspace call).
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one
 * GPU (different streams or threads without ordering between them) race and
 * give undefined results; calls ordered on one stream are fine. */
int32_t mla_decode_partial_noalloc(const mla_decode_desc* desc, const void* q, const void* kv_pool,
                                   const int32_t* block_table, const int32_t* context_lens,
                                   const int32_t* topk_idx, int32_t shard_id, int32_t n_shards,
                                   void* o_partial, float* lse, uint32_t* err_word, void* stream);

/* The same for shards shard_begin .. shard_begin + shard_count - 1 of
 * n_shards in one launch (all shards of one cache emulated on one GPU).
 *   block_tables [shard_count][B][max_blocks]
 *   o_partials   [shard_count][B*Tq][H][512] out_dtype
 *   lses         [shard_count][B*Tq][H] f32
 * workspace_bytes >= mla_decode_workspace_size(desc, shard_count). */
int32_t mla_decode_partial_shards(const mla_decode_desc* desc, const void* q,
                                  const void* kv_pool, const int32_t* block_tables,
                                  const int32_t* context_lens, const int32_t* topk_idx,
                                  int32_t shard_begin, int32_t shard_count, int32_t n_shards,
                                  void* o_partials, float* lses, void* workspace,
                                  int64_t workspace_bytes, void* stream);

/* mla_decode_partial_shards for requests with different numbers of query
 * tokens (varlen decode, as multi-token prediction produces: "GLM-5.2 vLLM
 * Decode Context Parallelism", section "See why vLLM 0.26.0 fails" names the
 * varlen-decode boundary the DCP backend must accept).  Request b has
 * query_start_loc[b + 1] - query_start_loc[b] query tokens, query token t of
 * it sits at position L_b - (its count) + t and attends positions up to it;
 * a request may have none.
 *   query_start_loc  [batch + 1] int32 device, first 0, last n_query_tokens,
 *                    nondecreasing; otherwise the call raises
 *                    MLA_DEVERR_QUERY in the workspace error word and its
 *                    outputs are unspecified (every access stays in bounds)
 *   q                [n_query_tokens][H][576]
 *   topk_idx         [n_query_tokens][topk] or NULL (dense)
 *   o_partials       [shard_count][n_query_tokens][H][512]
 *   lses             [shard_count][n_query_tokens][H]
 * desc->q_len bounds the call's size: n_query_tokens <= batch * q_len
 * (else MLA_ERR_SHAPE), and mla_decode_workspace_size(desc, shard_count)
 * sizes its workspace as for the fixed form.  Rows of o_partials / lses
 * follow the query tokens; mla_lse_merge combines them as usual. */
int32_t mla_decode_partial_shards_varlen(const mla_decode_desc* desc, const void* q,
                                         const void* kv_pool, const int32_t* block_tables,
                                         const int32_t* context_lens,
                                         const int32_t* query_start_loc, int32_t n_query_tokens,
                                         const int32_t* topk_idx, int32_t shard_begin,
                                         int32_t shard_count, int32_t n_shards, void* o_partials,
                                         float* lses, void* workspace, int64_t workspace_bytes,
                                         void* stream);

/* LSE merge of n_parts partials ("GLM-5.2 vLLM Decode Context Parallelism",
 * sections "See why vLLM 0.26.0 fails" and "Frequently asked questions"):
 *   M = max_s lse[s]; w_s = exp(lse[s] - M);
 *   o_out = sum_s w_s o[s] / sum_s w_s;  lse_out = M + log(sum_s w_s);
 * rows whose parts all have LSE -inf give (0, -inf) (the neutral row of an
 * empty shard drops out).  A part with LSE -inf contributes nothing, whatever
 * its o values.
 *   o_parts   [n_parts][rows][dv] part_dtype (MLA_F32 or MLA_BF16)
 *   lse_parts [n_parts][rows] f32
 *   o_out     [rows][dv] out_dtype;  lse_out [rows] f32, or NULL
 * 1 <= n_parts <= 64, rows >= 0, dv in {512}. */
int32_t mla_lse_merge(int32_t n_parts, int64_t rows, int32_t dv, int32_t part_dtype,
                      const void* o_parts, const float* lse_parts, int32_t out_dtype,
                      void* o_out, float* lse_out, void* stream);

/* Localise global top-K indices to one shard ("GLM-5.2 vLLM Decode Context
 * Parallelism", section "Separate the backend merge from stable"):
 *   local_idx[i] = global_idx[i] div n_shards  if global_idx[i] >= 0 and
 *                                                global_idx[i] mod n_shards == shard_id
 *                = -1                           otherwise.
 * count >= 0 int32 entries; bit-exact. */
int32_t mla_localize_indices(const int32_t* global_idx, int64_t count, int32_t shard_id,
                             int32_t n_shards, int32_t* local_idx, void* stream);

/* Cache slots of new tokens under round-robin ownership ("How vLLM Serves
 * GLM-5.3 with Million-Token Contexts on 16 H200s", section "The core
 * design"): token i of request b = req_idx[i] at global position
 * p = positions[i] belongs to shard s = p mod n_shards as its local token
 * j = p div n_shards, stored in row j mod 64 of pool block
 * block_tables[s - shard_begin][b][j / 64].  For tokens owned by a shard in
 * shard_begin .. shard_begin + shard_count - 1:
 *   slot_mapping[i] = block * 64 + j mod 64
 * and for every other token -1: a token another rank owns, or padding
 * (p < 0, or b outside [0, batch)).  A table row too narrow for j, or a block
 * id outside [0, pool_blocks), gives -1 and sets MLA_DEVERR_BLOCK_TABLE in
 * the error word.  shard_count = 1 is the call one DCP rank makes;
 * shard_count = n_shards gives every token its owner's slot in one pool
 * shared by all shards (the one-GPU emulation).
 *   req_idx, positions  [n_tokens] int32
 *   block_tables        [shard_count][batch][max_blocks] int32
 *   slot_mapping        [n_tokens] int64 (output, 8-byte aligned)
 *   workspace           NULL, or a buffer whose first 32-bit word is the
 *                       sticky device error word (as for decode)
 * Bit-exact integer work.  n_tokens >= 0; batch, max_blocks, pool_blocks >= 1. */
int32_t mla_dcp_slot_mapping(const int32_t* req_idx, const int32_t* positions, int64_t n_tokens,
                             const int32_t* block_tables, int32_t batch, int32_t max_blocks,
                             int64_t pool_blocks, int32_t shard_begin, int32_t shard_count,
                             int32_t n_shards, int64_t* slot_mapping, void* workspace,
                             void* stream);

/* Write new tokens into the paged pool at their slots.  Token i's 576 values
 * (512 latent, then 64 rope) go to row slot_mapping[i] in kv_dtype's row
 * format (see "Layouts"); a negative slot writes nothing.  With DCP a
 * negative slot marks a token whose KV another rank owns: ownership
 * suppresses only the cache write, never the token's query work, which this
 * call does not touch ("GLM-5.2 vLLM Decode Context Parallelism", section
 * "Keep the current-main correctness blocker visible").  A slot at or past
 * pool_blocks * 64 writes nothing and sets MLA_DEVERR_SLOT.
 *   kv_new        [n_tokens][576] src_dtype (MLA_F32 or MLA_BF16), 16-byte aligned
 *   slot_mapping  [n_tokens] int64, 8-byte aligned; non-negative slots must
 *                 be distinct (a repeated slot leaves that row unspecified)
 *   kv_pool       [pool_blocks][64][row] kv_dtype, 16-byte aligned
 *   workspace     NULL, or a buffer whose first 32-bit word is the error word
 * Conversions: f32 -> bf16 rounds to nearest even; bf16 -> f32 is exact.
 * MLA_FP8_DS rows (the pages' packed fp8 cache, "GLM-5.2 vLLM Decode Context
 * Parallelism", section "Understand the cache-copy opportunity"; the
 * quantiser itself is not on the pages): per 128-dim group g,
 *   scale_g = max |x| / 448 in float32 (1 if the group is all zero),
 *   code[d] = E4M3FN(x[d] / scale_g) rounded to nearest even, saturating at
 *             +-448 (float32 IEEE division),
 * and the rope part is stored as bf16.  Inputs must be finite.  Codes,
 * scales and rows are bit-exact functions of the input.  n_tokens >= 0. */
int32_t mla_kv_write(const void* kv_new, int32_t src_dtype, int64_t n_tokens,
                     const int64_t* slot_mapping, int32_t kv_dtype, void* kv_pool,
                     int64_t pool_blocks, void* workspace, void* stream);

/* mla_dcp_slot_mapping and mla_kv_write in one launch: each token's slot is
 * computed from req_idx, positions and the shards' block tables exactly as
 * mla_dcp_slot_mapping defines it, and the token's row is written there as
 * mla_kv_write defines it; tokens no shard in the range owns (or padding)
 * are skipped without reading their source row.  Table errors set
 * MLA_DEVERR_BLOCK_TABLE.  Arguments as in those two calls; no slot array
 * is read or written.  Knowing the share of tokens its shards own, the call
 * sizes its grid so each wave gathers about eight written tokens. */
int32_t mla_dcp_kv_write(const void* kv_new, int32_t src_dtype, const int32_t* req_idx,
                         const int32_t* positions, int64_t n_tokens, const int32_t* block_tables,
                         int32_t batch, int32_t max_blocks, int32_t shard_begin, int32_t shard_count,
                         int32_t n_shards, int32_t kv_dtype, void* kv_pool, int64_t pool_blocks,
                         void* workspace, void* stream);

/* Local top-K of the sparse indices on shards shard_begin .. shard_begin +
 * shard_count - 1: for every request b and query token t, the topk best
 * positions the shard owns in the token's causal prefix (positions 0 ..
 * L_b - Tq + t) by indexer score ("GLM-5.2 vLLM Decode Context Parallelism",
 * section "Understand the cache-copy opportunity": sparse index top-K;
 * "How vLLM Serves GLM-5.3 with Million-Token Contexts on 16 H200s", section
 * "Why conventional TP and DP fall short": the indexer scores earlier
 * tokens, sparse attention selects a fixed set).  Order: larger score first,
 * equal scores by lower position (+0 and -0 equal); the selection is unique.
 *   scores      [shard_count][B][Tq][row_stride] f32: entry j of shard s is the
 *               score of global position j * n_shards + s (what a DCP rank
 *               holds for its own tokens); finite or -inf
 *   cand_idx    [shard_count][B][Tq][topk] int32 GLOBAL positions, ascending,
 *               padded with -1 when the shard owns fewer than topk
 *   cand_score  [shard_count][B][Tq][topk] f32, the scores of cand_idx (-0 as
 *               +0; -inf
 *               for padding)
 *   workspace   NULL or a buffer whose first 32-bit word is the error word:
 *               a row_stride shorter than a shard's visible prefix sets
 *               MLA_DEVERR_SCORES and only the first row_stride entries count
 * 1 <= row_stride <= 393216 (the selection keeps a bitmap of the row's
 * positions in LDS beside its other state; MLA_ERR_SHAPE above), topk >= 1,
 * scores 4-byte aligned.  Bit-exact. */
int32_t mla_topk_local(const float* scores, int64_t row_stride, const int32_t* context_lens,
                       int32_t batch, int32_t q_len, int32_t topk, int32_t shard_begin,
                       int32_t shard_count, int32_t n_shards, int32_t* cand_idx, float* cand_score,
                       void* workspace, void* stream);

/* mla_topk_local for requests with different numbers of query tokens (the
 * varlen-decode layout that multi-token prediction produces; "GLM-5.2 vLLM
 * Decode Context Parallelism", section "See why vLLM 0.26.0 fails": the DCP
 * backend must accept it).  Request b holds query tokens query_start_loc[b]
 * .. query_start_loc[b + 1] - 1; with c of them, its token t is the fixed
 * form's token t with Tq = c and selects among positions 0 .. L_b - c + t.
 *   query_start_loc  [batch + 1] int32 on the device: 0, non-decreasing,
 *                    last entry n_q
 *   scores           [shard_count][n_q][row_stride] f32 (as mla_topk_local,
 *                    one row per query token)
 *   cand_idx         [shard_count][n_q][topk] int32 GLOBAL positions
 *   cand_score       [shard_count][n_q][topk] f32
 *   workspace        NULL or the error word: offsets that are not such a
 *                    partition set MLA_DEVERR_QUERY and the tokens that
 *                    cannot be placed select nothing (all -1)
 * Bounds, order and exactness as mla_topk_local.  The merge takes the
 * n_q rows as they are (mla_topk_merge with rows = n_q). */
int32_t mla_topk_local_varlen(const float* scores, int64_t row_stride, const int32_t* context_lens,
                              const int32_t* query_start_loc, int32_t batch, int32_t n_q, int32_t topk,
                              int32_t shard_begin, int32_t shard_count, int32_t n_shards,
                              int32_t* cand_idx, float* cand_score, void* workspace, void* stream);

/* Merge of candidate lists into the global top-K: for each row, the topk
 * best of the union of the n_lists lists (same order as mla_topk_local), as
 * ascending positions padded with -1.  Every global top-K position is in its
 * owner's local top-K, so merging the shards' mla_topk_local lists gives the
 * selection over the whole prefix.
 *   cand_idx, cand_score  [n_lists][rows][cand_k] (entries with index < 0 are
 *                         padding; positions must be distinct within a row)
 *   topk_idx              [rows][topk] int32 (the sparse decode's top-K input)
 * 1 <= n_lists, 1 <= topk <= 8192, n_lists * cand_k <= 2^18. */
int32_t mla_topk_merge(const int32_t* cand_idx, const float* cand_score, int32_t n_lists, int64_t rows,
                       int32_t cand_k, int32_t topk, int32_t* topk_idx, void* stream);

/* Read the device error word of a workspace: waits for `stream`, then copies
 * the word to *code_out (0 = no error; else MLA_DEVERR_* bits).  A block
 * table narrower than a request's local length is reported here as
 * MLA_DEVERR_BLOCK_TABLE instead of being copied past its end: the table
 * width a shard needs depends on the DCP factor, and a width mismatch is a
 * failure signature of its own ("GLM-5.2 vLLM Decode Context Parallelism",
 * section "Measure capacity and service behavior").  Host function; the
 * workspace pointer is a device pointer. */
int32_t mla_get_device_error(const void* workspace, int32_t* code_out, void* stream);

/* Enqueue a reset of the device error word to 0 on `stream`. */
int32_t mla_clear_device_error(void* workspace, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DCP_H */
