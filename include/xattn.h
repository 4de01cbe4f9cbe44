/*
 * xattn.h - staged beam-search decode attention over a split KV cache,
 * hand-written HIP kernels for AMD Instinct MI355X (gfx950, CDNA4).
 *
 * The method (xGR page, "xGR: Atendimento de Recomendação Generativa Eficiente
 * em Escala", section 2.1 xAttention): the KV cache of a generative-recommendation
 * request is split in two. The Shared cache holds the prompt (user history),
 * computed once at prefill and read once for all beams of the request. The
 * Non-Shared cache holds only the tokens generated at each decode step,
 * managed per token (no blocks), so a beam that branches copies nothing.
 * Attention is computed in stages: a Shared stage and a Non-Shared stage each
 * produce local scores and max/sum statistics; a Merge stage combines them
 * with online softmax. Updates to the Non-Shared cache happen in place through
 * direct indices with no read-before-write hazard. Section 1 of the same page
 * states the problem this removes (per-beam reloads of the shared prompt and
 * block copies on branching).
 *
 * CONVENTIONS
 *  - Every pointer argument named as device memory must point to memory the
 *    caller allocated on the current HIP device. Apart from the step-graph
 *    create/destroy calls, the library never allocates, frees or
 *    synchronizes; it only enqueues kernels on `stream` (a hipStream_t;
 *    NULL = the null stream) and returns.
 *  - Every condition the host can check is checked before anything is
 *    launched; on error nothing is enqueued. The contents of device arrays
 *    (lengths, offsets, slot indices, parents) are trusted: out-of-range
 *    values are undefined behaviour.
 *  - Results are deterministic: split counts depend only on the dims and
 *    partial results are always combined in the same order, so repeated calls
 *    give identical bits (a counter only decides which workgroup combines).
 *
 * NOTATION
 *  R requests; B beam width; beam n = r*B + b (N_b = R*B beams);
 *  H_q query heads, H_kv kv heads, G = H_q / H_kv, query head q reads kv head
 *  q / G; D head dim; P_r prompt (prefix) length of request r; L_r the number
 *  of generated tokens of request r, counting the current step's own token.
 *
 * DEVICE LAYOUTS (row-major, element type per dims.dtype unless stated)
 *  q            [N_b][H_q][D]
 *  k_shared     [H_kv][n_ptok][D]   request r owns tokens
 *  v_shared     [H_kv][n_ptok][D]     [prefix_off[r], prefix_off[r] + P_r);
 *                                     several requests may alias one range
 *  prefix_off   [R] int64, prefix_len [R] int32 (0 <= P_r <= max_prefix_len)
 *  k_pool       [num_slots][H_kv][D]  Non-Shared pool, one slot per token
 *  v_pool       [num_slots][H_kv][D]
 *  slot_table   [N_b][max_unshared_len] int32; row n valid on [0, L_r)
 *  unshared_len [R] int32 (0 <= L_r <= max_unshared_len)
 *  o            [N_b][H_q][D] float32 (normalized attention output)
 *  lse          [N_b][H_q] float32, natural-log sum of exp(scale * q.k) over
 *               the part's keys; -inf (and o = 0) for an empty part.
 */
#ifndef XATTN_H
#define XATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  XATTN_OK = 0,
  XATTN_ERR_INVALID_ARG = 1, /* null pointer, bad size, inconsistent dims */
  XATTN_ERR_UNSUPPORTED = 2, /* head_dim / dtype / shape outside the built kernels */
  XATTN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than xattn_workspace_size */
  XATTN_ERR_HIP = 4          /* a HIP launch reported an error */
} xattn_status;

typedef enum { XATTN_F32 = 0, XATTN_BF16 = 1 } xattn_dtype;

/* Host-side sizes. All arrays are passed separately as device pointers. */
typedef struct {
  int32_t num_requests;     /* R >= 0 */
  int32_t beam_width;       /* B >= 1 */
  int32_t num_q_heads;      /* H_q >= 1, a multiple of num_kv_heads */
  int32_t num_kv_heads;     /* H_kv >= 1 */
  int32_t head_dim;         /* D: 64 or 128 */
  int32_t max_prefix_len;   /* >= every prefix_len[r]; sizes the prefix split plan.
                               max_prefix_len * head_dim * element bytes must stay
                               below 2^31 (else XATTN_ERR_UNSUPPORTED) */
  int32_t max_unshared_len; /* T_max >= 1: slot-table row stride, >= every unshared_len[r] */
  int32_t dtype;            /* xattn_dtype of q and every K/V buffer */
  int64_t num_slots;        /* capacity of k_pool / v_pool in tokens */
  int64_t num_prefix_tokens;/* n_ptok: token extent of k_shared / v_shared */
  float scale;              /* softmax scale applied to q.k (normally 1/sqrt(D)); must be
                               finite and > 0, else XATTN_ERR_INVALID_ARG */
  int32_t prefix_splits;    /* 0 = automatic; else force this many prefix splits */
  int32_t unshared_splits;  /* 0 = automatic; else force this many Non-Shared splits
                               (forces the Non-Shared part out of the fused epilogue) */
  int32_t rows_per_block;   /* 0 = automatic; else 32, 64 or 128 query rows per
                               Shared-stage workgroup (bf16 MFMA path) */
  int32_t pipeline_stages;  /* 0 = automatic; else 2 or 4 K/V tiles staged in LDS */
  int32_t key_groups;       /* 0 = automatic; else 1, 2 or 4 wavefront groups
                               per Shared-stage workgroup that split the keys of
                               the same query rows (merged in LDS). Two groups
                               with 2 stages take alternate 64-key tiles, with 4
                               stages the two 32-key halves of every tile. Four
                               groups (head_dim 128, 32 or 64 rows, 2 stages
                               only; else XATTN_ERR_UNSUPPORTED, or
                               XATTN_ERR_INVALID_ARG for 4 stages) take the
                               32-key halves of two 64-key tiles per step */
  int32_t prompts_disjoint; /* 0 or 1 (else XATTN_ERR_INVALID_ARG). 1: the caller
                               guarantees that no two requests' prompt ranges
                               [prefix_off[r], prefix_off[r] + P_r) overlap. A
                               prompt that one workgroup alone reads (a single
                               tile of query rows) is then loaded with
                               non-temporal loads, which stream it past the
                               caches; with aliased prompts (0) other requests
                               find it in the caches, so the default policy
                               stays. A cache hint only: results are identical. */
} xattn_dims;

/* Launch plan chosen for a dims (introspection for tests and tuning). */
typedef struct {
  int32_t rows_per_block;   /* query rows per Shared-stage workgroup (32 per wave) */
  int32_t row_tiles;        /* ceil(B*G / rows_per_block) per (request, kv head) */
  int32_t prefix_splits;    /* key-range splits of the prompt */
  int32_t prefix_chunk;     /* keys per split (a multiple of 64) */
  int32_t unshared_splits;  /* 0 = Non-Shared part fused into the Shared epilogue */
  int32_t unshared_chunk;   /* generated tokens per Non-Shared split */
  int32_t partials;         /* (O, lse) partial slots in the workspace */
  int32_t mfma;             /* 1 = bf16 MFMA Shared stage, 0 = vector-ALU path */
  int32_t launches;         /* kernel launches per call */
  int32_t pipeline_stages;  /* K/V tiles staged in LDS (MFMA path) */
  int32_t key_groups;       /* wavefront groups splitting each workgroup's keys */
} xattn_plan;

/*
 * Workspace bytes needed by a call. which: 0 = xattn_shared_stage,
 * 1 = xattn_unshared_stage, 2 = xattn_decode, 3 = xattn_append_decode. A
 * size of 0 means the call needs no workspace (a null workspace pointer is
 * then allowed).
 * The workspace (device memory, 16-byte aligned, owned by the caller) starts
 * with a block of split counters that must be zero-filled before the buffer's
 * first use; every call returns them to zero, so a buffer is reusable by any
 * later call. Calls that may run at the same time (e.g. on different streams)
 * must not share a workspace.
 */
xattn_status xattn_workspace_size(const xattn_dims* dims, int which, size_t* bytes);

/* The plan xattn_decode (which = 2), xattn_shared_stage (0) or
 * xattn_unshared_stage (1) will use for these dims. */
xattn_status xattn_get_plan(const xattn_dims* dims, int which, xattn_plan* plan);

/*
 * Shared stage (xGR page, section 2.1, staged computation): for every request
 * r and kv head h, all B*G query rows attend to the request's prompt keys
 * [prefix_off[r], prefix_off[r] + P_r) of k_shared / v_shared. The prompt KV
 * of a (request, kv head) is streamed from HBM once for all its beams.
 * Writes o_shared [N_b][H_q][D] and lse_shared [N_b][H_q] (float32, device).
 * bf16 inputs run on bf16 MFMA with fp32 accumulation; fp32 inputs on the
 * vector ALUs.
 */
xattn_status xattn_shared_stage(const xattn_dims* dims, const void* q, const void* k_shared,
                                const void* v_shared, const int64_t* prefix_off,
                                const int32_t* prefix_len, float* o_shared, float* lse_shared,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Non-Shared stage (xGR page, section 2.1, separate KV cache and token-granular
 * management): every beam n attends to its own generated tokens, the pool
 * slots slot_table[n][0 .. L_r). Writes o_unshared / lse_unshared (float32).
 */
xattn_status xattn_unshared_stage(const xattn_dims* dims, const void* q, const void* k_pool,
                                  const void* v_pool, const int32_t* slot_table,
                                  const int32_t* unshared_len, float* o_unshared,
                                  float* lse_unshared, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * Merge stage (xGR page, section 2.1: online softmax over the stages' max/sum
 * statistics): for each of `rows` rows of `head_dim` floats,
 *   lse = log(exp(lse_a) + exp(lse_b)),
 *   o   = exp(lse_a - lse) * o_a + exp(lse_b - lse) * o_b,
 * with an empty part (lse = -inf) contributing nothing and two empty parts
 * giving o = 0, lse = -inf. All pointers are float32 device memory.
 * o_out may equal o_a or o_b (in place); lse_out may be NULL or equal
 * lse_a / lse_b.
 */
xattn_status xattn_merge(int64_t rows, int32_t head_dim, const float* o_a, const float* lse_a,
                         const float* o_b, const float* lse_b, float* o_out, float* lse_out,
                         void* stream);

/*
 * Fused decode attention: Shared stage + Non-Shared stage + Merge in one pass
 * (the measured call). The Non-Shared part runs in the Shared stage's
 * epilogue when the plan fuses it; otherwise it runs as its own split work
 * and the partials are combined by the log-sum-exp rule: when the plan gives
 * the Non-Shared tokens a vector pass of their own with at most 8 splits
 * (long generated tails), that pass folds the prompt partials in and writes
 * o and lse itself; in every other split plan one reduction merges all
 * partials. Writes o [N_b][H_q][D] and, if lse is not NULL, lse [N_b][H_q].
 */
xattn_status xattn_decode(const xattn_dims* dims, const void* q, const void* k_shared,
                          const void* v_shared, const int64_t* prefix_off,
                          const int32_t* prefix_len, const void* k_pool, const void* v_pool,
                          const int32_t* slot_table, const int32_t* unshared_len, float* o,
                          float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * In-place token-granular append of one decode step (xGR page, section 2.1,
 * in-place updates through direct indices without read-before-write
 * hazards; section 1, block copies on branching are what this avoids).
 * For every request r with active[r] != 0 (active may be NULL = all) and
 * t = unshared_len[r] < max_unshared_len, and every new beam b:
 *   slot                  = slot_base[r] + t*B + b
 *   k_pool[slot], v_pool[slot] <- k_new[r*B + b], v_new[r*B + b]   ([H_kv][D] each)
 *   table_out[r*B+b][0..t) <- table_in[r*B + parent[r*B+b]][0..t)  (t > 0 only)
 *   table_out[r*B+b][t]    <- slot
 * then unshared_len[r] += 1. Columns beyond t are not written. parent values
 * are request-local beam indices in [0, B); they are ignored at t = 0.
 * table_out may equal table_in: every parent row is read before any row is
 * written, so the in-place result equals the out-of-place one.
 * k_new / v_new: [N_b][H_kv][D] (dims.dtype); parent [N_b] int32;
 * slot_base [R] int64; active [R] uint8 or NULL; tables [N_b][T_max] int32;
 * unshared_len [R] int32 (read, then incremented). Needs no workspace.
 * Slots must lie in [0, num_slots). A request that takes no token (inactive,
 * or its row full: t == max_unshared_len) keeps its length and pool; with a
 * separate table_out its rows are copied there (columns 0..t-1), so that
 * table_out is a complete table either way.
 * One kernel launch: while it runs, its workgroups count their arrivals in
 * bits 20 and up of unshared_len, so lengths must stay below 2^20 and nothing
 * else may read unshared_len during the call. XATTN_ERR_UNSUPPORTED if
 * max_unshared_len >= 2^20 or one request would need more than 2047
 * workgroups (very large beam_width * max_unshared_len).
 */
xattn_status xattn_cache_append(const xattn_dims* dims, const void* k_new, const void* v_new,
                                const int32_t* parent, const int64_t* slot_base,
                                const uint8_t* active, void* k_pool, void* v_pool,
                                const int32_t* table_in, int32_t* table_out,
                                int32_t* unshared_len, void* stream);

/*
 * One decode step of a layer in one call: xattn_cache_append of the step's
 * new K/V rows, then xattn_decode over the updated cache (xGR page, section
 * 2.1: the token-granular in-place update and the staged attention of the
 * same step). Arguments are those of the two calls; the decode reads
 * table_out, which must be a different buffer from table_in (the ping-pong
 * form: the next step passes this table_out as its table_in). The result is
 * bit for bit that of the two calls in order.
 * When the decode plan is a single launch (bf16 MFMA path, one prompt range,
 * Non-Shared tokens folded in) the append is folded into that launch: each
 * attention workgroup counts its arrival on unshared_len as the append does,
 * reads every beam's older tokens through its parent's row of table_in and
 * its new token straight from k_new / v_new, and writes the pool rows,
 * table_out rows and lengths of the beams it owns; arrivals are counted per
 * (request, kv head) in the workspace (which = 3 in xattn_workspace_size),
 * then per request on unshared_len. When the plan gives the Non-Shared
 * tokens a vector pass of their own (long generated tails, bf16) the append
 * folds into the MFMA prompt pass instead: prompt split 0's workgroups write
 * the pool rows, table_out rows and lengths (the prompt pass reads neither
 * the pool nor the tables), the Non-Shared pass after it reads table_out, and
 * its arrival counters are the head of the decode's workspace. Otherwise the
 * two calls are made in order, with the decode's workspace. Same limits and
 * errors as the two calls, and XATTN_ERR_INVALID_ARG if table_out ==
 * table_in.
 */
xattn_status xattn_append_decode(const xattn_dims* dims, const void* q, const void* k_shared,
                                 const void* v_shared, const int64_t* prefix_off,
                                 const int32_t* prefix_len, const void* k_new, const void* v_new,
                                 const int32_t* parent, const int64_t* slot_base,
                                 const uint8_t* active, void* k_pool, void* v_pool,
                                 const int32_t* table_in, int32_t* table_out,
                                 int32_t* unshared_len, float* o, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * xattn_append_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, which comes instead
 * from a fixed array of 32 MiB in the library's device memory (one per GPU,
 * held until the process ends; found once per device on the first call).
 * Nothing is allocated or freed. The split counters at its head are cleared
 * by a small fill kernel on `stream` before the call's own launch.
 * Every call on one GPU shares that GPU's array: calls that may overlap on a
 * GPU (different streams, threads) race and must not be issued. Results are
 * those of xattn_append_decode with a workspace of xattn_workspace_size(dims,
 * 3) bytes. XATTN_ERR_WORKSPACE if that size exceeds 32 MiB; otherwise the
 * errors of xattn_append_decode, and XATTN_ERR_HIP if the array's address
 * cannot be found.
 */
xattn_status xattn_append_decode_static(const xattn_dims* dims, const void* q, const void* k_shared,
                                        const void* v_shared, const int64_t* prefix_off,
                                        const int32_t* prefix_len, const void* k_new, const void* v_new,
                                        const int32_t* parent, const int64_t* slot_base,
                                        const uint8_t* active, void* k_pool, void* v_pool,
                                        const int32_t* table_in, int32_t* table_out,
                                        int32_t* unshared_len, float* o, float* lse, void* stream);

/*
 * Beam-search survivor selection for one decode step (xGR page, section 2.2
 * xBeam: the Top-K sequences are chosen from the pool of every live beam's
 * candidates; since a beam's candidates come sorted, a walk over the pool
 * with a global min-heap stops a beam at its first candidate below the heap
 * minimum). Per request r, the pool holds beam_width * top_k candidates
 * (b, k) with score = beam_score[r][b] + logprob[r][b][k], added in float32.
 * The n_out best by (score descending, pool index b * top_k + k ascending;
 * -0.0 equals +0.0) are written in that order:
 *   parent[r][i]    = b            (feeds xattn_cache_append's parent array)
 *   token_out[r][i] = token[r][b][k]
 *   score_out[r][i] = the score
 * beam_score [R][beam_width] float32; logprob [R][beam_width][top_k]
 * float32, every row non-increasing along k (required: the walk stops a
 * beam early); scores finite or -inf (no NaN); token [R][beam_width][top_k]
 * int32; outputs [R][n_out]. One workgroup per request, no workspace.
 * XATTN_ERR_INVALID_ARG for null pointers or n_out > beam_width * top_k;
 * XATTN_ERR_UNSUPPORTED if beam_width > 8192, n_out > 4096 or
 * top_k > 8192 - n_out. n_out = 0 or num_requests = 0 enqueue nothing.
 */
xattn_status xattn_beam_topk(int32_t num_requests, int32_t beam_width, int32_t top_k,
                             int32_t n_out, const float* beam_score, const float* logprob,
                             const int32_t* token, int32_t* parent, int32_t* token_out,
                             float* score_out, void* stream);

/*
 * COMPARISON BASELINE: PagedAttention-style per-beam decode attention (xGR
 * page, section 1: serving systems in the PagedAttention mould treat each
 * beam as an independent sequence, so the shared prompt is loaded again for
 * every beam and branching beams copy their partially filled blocks). It
 * computes the same o / lse as xattn_decode for a beam whose sequence is its
 * prompt followed by its own generated tokens, but from a block-paged cache:
 *   k_cache, v_cache  [num_blocks][H_kv][16][D] bf16 (16-token blocks)
 *   block_table       [N_b][max_blocks] int32: beam n's i-th block
 *   seq_len           [N_b] int32, <= max_seq_len <= 16 * max_blocks
 * Uses dims.num_requests, beam_width, num_q_heads, num_kv_heads, head_dim,
 * scale; dtype must be XATTN_BF16 (else XATTN_ERR_UNSUPPORTED). Sequences
 * longer than 512 tokens are split in partitions merged in a second launch;
 * that needs xattn_paged_workspace_size bytes of workspace (0 otherwise).
 */
xattn_status xattn_paged_workspace_size(const xattn_dims* dims, int32_t max_seq_len, size_t* bytes);
xattn_status xattn_paged_decode(const xattn_dims* dims, int32_t max_seq_len, const void* q,
                                const void* k_cache, const void* v_cache,
                                const int32_t* block_table, int32_t max_blocks,
                                const int32_t* seq_len, float* o, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream);
/*
 * COMPARISON BASELINE: copy whole cache blocks (every kv head) src[i] ->
 * dst[i], i < n, in both k_cache and v_cache ([num_blocks][H_kv][16][D]
 * bf16): the copy-on-write a branching beam needs in a block-paged cache.
 * Destination blocks must be distinct and not sources.
 */
xattn_status xattn_paged_copy_blocks(const xattn_dims* dims, void* k_cache, void* v_cache,
                                     const int32_t* src, const int32_t* dst, int32_t n,
                                     void* stream);

/*
 * Multi-layer decode step as one HIP graph (xGR page, section 2.3 xSchedule:
 * device work is captured once into a static graph and submitted as a whole,
 * cutting kernel-launch overhead and CPU involvement; the xLLM page's engine
 * layer does the same with dimension parameters and reports a throughput
 * gain for smaller models in its ablations). At the GR decode sizes the
 * per-call host launch path costs more than the kernel itself.
 *
 * Each layer is self-contained: its own pool, slot tables and lengths. The
 * step first runs the optional survivor selection (xattn_beam_select, the
 * xattn_beam_topk arguments; its parent output is what the layers' appends
 * normally read), then, for every layer in order, xattn_cache_append
 * (skipped when k_new is NULL) and xattn_decode on the table the append
 * wrote (table_out), with the arguments below exactly as those calls take
 * them. With separate tables (table_in != table_out) and no decode_begin
 * event, the pair is captured as one xattn_append_decode call, which folds
 * the append into the decode launch where the plan allows.
 * Positions are read from device memory when the graph runs, so one graph
 * serves every decode step: refill the candidates, q, k_new and v_new in
 * place and launch it again. If decode_begin / decode_end are not NULL (hipEvent_t
 * created with timing enabled), they are captured as external event-record
 * nodes around the layer's decode, recorded on every launch; a HIP runtime
 * that cannot capture external event records (the one PyTorch 2.10 ships
 * for ROCm 7.0 cannot) makes the create call fail with XATTN_ERR_HIP.
 */
typedef struct {
  xattn_dims dims;
  const void* k_new;         /* NULL: no append in this layer */
  const void* v_new;
  const int32_t* parent;
  const int64_t* slot_base;
  const uint8_t* active;
  const int32_t* table_in;
  int32_t* table_out;        /* also the decode's slot table */
  int32_t* unshared_len;
  const void* q;
  const void* k_shared;
  const void* v_shared;
  const int64_t* prefix_off;
  const int32_t* prefix_len;
  void* k_pool;
  void* v_pool;
  float* o;
  float* lse;                /* may be NULL */
  void* workspace;
  size_t workspace_bytes;
  void* decode_begin;        /* hipEvent_t or NULL */
  void* decode_end;          /* hipEvent_t or NULL */
} xattn_layer_step;

typedef struct {
  int32_t num_requests;
  int32_t beam_width;
  int32_t top_k;
  int32_t n_out;
  const float* beam_score;
  const float* logprob;
  const int32_t* token;
  int32_t* parent;
  int32_t* token_out;
  float* score_out;
} xattn_beam_select;

typedef struct xattn_step_graph xattn_step_graph;  /* opaque */

/*
 * Capture the step (select may be NULL: no selection) for n_layers >= 0
 * layers (at least one of the two) and instantiate it. Every
 * argument is validated as the eager calls validate theirs; on any error
 * nothing is kept and *graph is left NULL. This call (and only this one, with
 * destroy) allocates: the graph, its executable form and a capture stream.
 * XATTN_ERR_HIP if capture or instantiation fails.
 */
xattn_status xattn_step_graph_create(const xattn_beam_select* select,
                                     const xattn_layer_step* layers, int32_t n_layers,
                                     xattn_step_graph** graph);
/* Enqueue one step on `stream`. The graph's buffers must not be in use by
 * other work on other streams meanwhile. */
xattn_status xattn_step_graph_launch(xattn_step_graph* graph, void* stream);
/* Release the graph (NULL is allowed). The caller makes sure no launch of it
 * is still running. */
xattn_status xattn_step_graph_destroy(xattn_step_graph* graph);

/*
 * HOST-SIDE batch former (Feather page, "Requests of a Feather Must Flock
 * Together", Metodologia 1: requests as cumulative hashes over fixed-size
 * token blocks, a working set of the active batch's hashes and a min-heap of
 * waiting requests by missing count, best candidate in O(log W)). Groups of
 * sequences it puts together share a prefix, which is what xattn_decode
 * serves as one request with the sequences as its beams.
 *  - A request's full blocks are hashed cumulatively (a trailing partial
 *    block is ignored); block i is covered when an active request has the
 *    same tokens over blocks 0..i. missing = full blocks not covered.
 *  - best: the waiting request with the fewest missing blocks, ties to the
 *    earliest inserted; (-1, -1) when none waits.
 *  - form_batch: if nothing is active, admit the earliest waiting request;
 *    then admit the best while its missing count <= max_missing and fewer
 *    than max_batch requests are active. Writes the admitted ids, in order,
 *    to out_ids (room for max_batch) and their number to *out_n.
 * Request ids are caller-chosen, >= 0 and unique among live requests.
 * admit takes a waiting request, complete an active one (which is then
 * forgotten); anything else is XATTN_ERR_INVALID_ARG. Runs on the host and
 * allocates host memory; one structure must not be used by two threads at
 * once.
 */
typedef struct xattn_cht xattn_cht;  /* opaque */
xattn_status xattn_cht_create(int32_t block_size, xattn_cht** cht);
xattn_status xattn_cht_destroy(xattn_cht* cht);
xattn_status xattn_cht_insert(xattn_cht* cht, int64_t request_id, const int32_t* tokens,
                              int64_t n_tokens);
xattn_status xattn_cht_best(xattn_cht* cht, int64_t* request_id, int64_t* missing);
xattn_status xattn_cht_admit(xattn_cht* cht, int64_t request_id);
xattn_status xattn_cht_complete(xattn_cht* cht, int64_t request_id);
xattn_status xattn_cht_form_batch(xattn_cht* cht, int32_t max_batch, int64_t max_missing,
                                  int64_t* out_ids, int32_t* out_n);

/*
 * MEASUREMENT UTILITY (not part of the attention path): reads `bytes` of
 * device memory at src once, with 16-byte non-temporal vector loads spread
 * over every CU (eight in flight per thread; the fastest of the forms tried),
 * and discards the data. Timing it gives the practical HBM read ceiling that
 * the attention kernels' bandwidth figures are read against (xGR page,
 * section 4: the baseline kernel's memory pipeline is reported busy most of
 * the time, so the attainable bandwidth is the yardstick; the 8 TB/s of the
 * data sheet is not reachable by any kernel). src must be 16-byte aligned
 * and bytes a multiple of 16 (else XATTN_ERR_INVALID_ARG); sink is one
 * device uint32 that the kernel may overwrite with a meaningless value.
 * bytes = 0 enqueues nothing.
 */
xattn_status xattn_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Human-readable name of a status code (static storage). */
const char* xattn_status_string(xattn_status status);

#ifdef __cplusplus
}
#endif

#endif /* XATTN_H */
