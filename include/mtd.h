/*
 * mtd.h - paged causal grouped-query attention for a Qwen3-style decoder on AMD MI355X (gfx950).
 *
 * The decoder these kernels serve is the Qwen3 text decoder of an audio LLM: 28 layers, hidden size
 * 1024, grouped-query attention with 16 query heads over 8 key/value heads ("Optimizing ASR Models
 * to Transcribe 90-Minute Multi-Speaker Audio", section ASR Model Primer, component table; the
 * "MOSS-Transcribe-Diarize" cookbook, section Model Architecture).  head_dim is 128.  Its KV cache
 * holds tens of thousands of audio tokens per request (up to a 128K context, cookbook section Model
 * Architecture).  Three operations carry the attention work:
 *
 *   mtd_kv_append           write the K/V rows of new tokens into their cache pages
 *   mtd_attn_prefill_chunk  causal attention of one prefill chunk over the paged cache
 *                           ("Optimizing ASR Models ...", section Chunked Prefill for Long Audio:
 *                           4096-token pieces, each attending to everything before it and to
 *                           itself causally)
 *   mtd_attn_decode         one query token per request over that request's whole cache, for a
 *                           batch of requests ("Optimizing ASR Models ...", section ASR Model
 *                           Primer, Autoregressive Decode, and section Batched Inference)
 *
 * and two linear maps sit on either side of them in every decoder layer:
 *
 *   mtd_qkv_proj            hidden states -> q, k, v of new tokens
 *   mtd_o_proj              attention output -> hidden states
 *
 * and mtd_attn_merge combines attention results computed over disjoint key ranges (a request's KV
 * split by sequence).
 *
 * Everything computed is exact softmax attention:
 *     s_j = scale * <q, k_j>  for visible keys j;  LSE = ln sum_j exp(s_j);  O = sum_j exp(s_j - LSE) v_j
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * ---------------------------------------------------------------------------------------------
 * Conventions shared by every call
 * ---------------------------------------------------------------------------------------------
 * Memory.  Every pointer argument is a DEVICE pointer (memory of the GPU that is current on the
 *   calling thread) unless the comment says "host".  The caller owns all memory; the library
 *   allocates none and keeps no state other than a per-thread error string and, per device, the
 *   compute-unit count it reads once to size launches.
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue work on it,
 *   in order, and never synchronise the host.
 * bf16.  bfloat16 values are 2-byte IEEE-754 binary32 upper halves.
 * Page layout.  K and V live in separate pools, each
 *       bf16 [num_pages][num_kv_heads][page_size][head_dim]   (row-major, contiguous),
 *   so the rows of one (page, KV head) form one contiguous block of page_size*head_dim*2 bytes.
 *   Logical token p of a request is stored at page block_table[p / page_size], slot p % page_size.
 * Block tables.  int32 [n][bt_stride], row r lists request r's physical page ids in logical order.
 *   Entries a call does not need are never read.
 * Alignment.  The pools, the query, key and value rows, the float32 outputs O and every workspace
 *   must be 16-byte aligned (the kernels move 16-byte vectors); else MTD_ERR_INVALID_ARG.  LSE
 *   arrays and int32 arrays need only their natural alignment.
 * Supported shape (this version).  num_q_heads = 16, num_kv_heads = 8, head_dim = 128,
 *   page_size = 64; anything else returns MTD_ERR_UNSUPPORTED.
 * Errors.  Every argument that lives on the host is checked before any work is enqueued; a failed
 *   check returns a negative MTD_ERR_* code, enqueues nothing and leaves all memory untouched.
 *   Values that live on the device (table entries, lengths, offsets) are trusted: if they are
 *   inconsistent with the sizes given on the host the results are unspecified, but no kernel reads
 *   or writes outside the pools, the inputs and the outputs.  Page ids outside [0, num_pages) are
 *   skipped: mtd_kv_append leaves such a token unwritten, and mtd_attn_decode and
 *   mtd_attn_prefill_chunk give each query attention over the keys of the valid pages it may see
 *   (a query that sees none gets O = 0 and LSE = -inf).
 *   A failed kernel launch returns MTD_ERR_HIP; mtd_last_error() gives the detail.
 */
#ifndef MTD_H
#define MTD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MTD_ABI_VERSION 8

/* Status codes. */
#define MTD_OK               0
#define MTD_ERR_INVALID_ARG (-1) /* null pointer, negative or zero size where one is required     */
#define MTD_ERR_UNSUPPORTED (-2) /* head count, head_dim or page size this version does not build */
#define MTD_ERR_CAPACITY    (-3) /* tokens beyond the block-table capacity or the 128K context    */
#define MTD_ERR_WORKSPACE   (-4) /* workspace missing or smaller than the required size           */
#define MTD_ERR_HIP         (-5) /* the HIP runtime reported an error (see mtd_last_error)        */

/* Longest KV a request may hold (128K context). */
#define MTD_MAX_CONTEXT 131072

/* One layer's paged KV cache.  The struct itself lives on the host; the pools on the device. */
typedef struct mtd_kv_layer {
  void*   k_pages;      /* device, bf16 [num_pages][num_kv_heads][page_size][head_dim]          */
  void*   v_pages;      /* device, same layout                                                   */
  int32_t num_pages;    /* > 0                                                                   */
  int32_t page_size;    /* tokens per page: 64                                                   */
  int32_t num_kv_heads; /* 8                                                                     */
  int32_t head_dim;     /* 128                                                                   */
} mtd_kv_layer_t;

/*
 * mtd_kv_append - store the K/V rows of new tokens in their pages.
 *
 * Prefill writes the prompt's keys and values into the KV cache and every decode step adds the
 * new token's ("Optimizing ASR Models ...", section ASR Model Primer: "LLM Prefill" builds the KV
 * cache, "Autoregressive Decode" extends it; cookbook section Inference Pipeline).
 *
 *   kv          host pointer to the layer's pools (pools are modified in place)
 *   k_new       bf16 [n_new][num_kv_heads][head_dim], the new keys, requests back to back
 *   v_new       bf16 [n_new][num_kv_heads][head_dim], the new values
 *   cu_new      int32 [n_req + 1], cu_new[0] = 0, nondecreasing, cu_new[n_req] <= n_new: request r
 *               owns new rows cu_new[r] .. cu_new[r+1]-1; rows at or past cu_new[n_req] belong to
 *               no request and are not written (a batch padded to a fixed size, as in a captured
 *               graph serving fewer requests than it was captured for)
 *   start_pos   int32 [n_req], logical position of request r's first new token
 *   block_tables, bt_stride   int32 [n_req][bt_stride]; entry (start_pos[r] + i) / page_size of
 *               row r must be valid for every new token i of request r
 *   n_req       >= 1;  n_new >= 0 (0 enqueues nothing)
 *
 * Effect: for every new token t of request r at position p = start_pos[r] + (t - cu_new[r]) and
 * every KV head g, the head_dim values of k_new[t][g] are copied bit for bit to
 * k_pages[block_tables[r][p / page_size]][g][p % page_size], and likewise for V.  No other byte of
 * the pools changes.  Positions at or beyond MTD_MAX_CONTEXT are skipped.
 */
int mtd_kv_append(const mtd_kv_layer_t* kv, const void* k_new, const void* v_new,
                  const int32_t* cu_new, const int32_t* start_pos, const int32_t* block_tables,
                  int32_t bt_stride, int32_t n_req, int32_t n_new, void* stream);

/*
 * mtd_attn_prefill_chunk - causal attention of one prefill chunk over the paged cache.
 *
 * Long prompts are prefilled in 4096-token chunks, one per scheduler step; each chunk attends to
 * all keys before it and to itself causally ("Optimizing ASR Models ...", section Chunked Prefill
 * for Long Audio; cookbook section Inference Pipeline).  A short prompt is one chunk with
 * prefix_len = 0 (one-shot prefill).  The chunk's own K/V must already be in the pages
 * (mtd_kv_append first, on the same stream).
 *
 *   q               bf16 [chunk_len][num_q_heads][head_dim], chunk query i is at absolute
 *                   position prefix_len + i and sees keys 0 .. prefix_len + i
 *   chunk_len       >= 1;  prefix_len >= 0;  prefix_len + chunk_len <= MTD_MAX_CONTEXT
 *   block_table     int32 [block_table_len], the request's page ids in logical order
 *   block_table_len host: capacity of block_table in entries; must be at least
 *                   ceil((prefix_len + chunk_len) / page_size), else MTD_ERR_CAPACITY
 *   num_q_heads     16;  scale > 0 and finite (1/sqrt(head_dim) for the Qwen3 decoder)
 *   workspace       NULL, or device scratch of at least mtd_attn_prefill_workspace_bytes(chunk_len,
 *                   num_q_heads, head_dim) bytes (else MTD_ERR_WORKSPACE), owned by the caller,
 *                   contents ignored on entry and unspecified on return.  With a workspace, the
 *                   causal work of the (128-position tile, KV head) items is rebalanced over the
 *                   compute units, and the parts of a split item are merged by log-sum-exp: with
 *                   at least as many items as compute units, tiles t and T-1-t (T tiles in the
 *                   chunk) share two workgroups that each take half of their combined keys;
 *                   with fewer, every item's keys run as two halves.  Without a workspace, each
 *                   item is one pass.  All give correct results; their bits differ.  Calls on
 *                   different streams need different workspaces.
 *   out             float32 [chunk_len][num_q_heads][head_dim], written
 *   lse             float32 [chunk_len][num_q_heads], written: natural-log sum of exp(s_j)
 */
int mtd_attn_prefill_chunk(const mtd_kv_layer_t* kv, const void* q, int32_t chunk_len,
                           int32_t prefix_len, const int32_t* block_table, int32_t block_table_len,
                           int32_t num_q_heads, float scale, void* workspace, size_t workspace_bytes,
                           float* out, float* lse, void* stream);

/*
 * mtd_attn_prefill_chunk_cus - mtd_attn_prefill_chunk on a budget of compute units, so that other
 * work of the same scheduler step can run beside it.
 *
 * The scheduler interleaves other requests' decode with the chunks of a long prompt ("Optimizing
 * ASR Models ...", section Chunked Prefill for Long Audio).  Prefill is bound by the matrix units
 * and decode by HBM, so the two overlap well only on separate compute units: with cu_budget > 0
 * (and below the device's CU count) and a workspace, each KV head's causal work (its position
 * tiles' key tiles, longest tile first, laid end to end) is cut into cu_budget / 8 equal ranges,
 * one workgroup of one CU each (fewer if a range would be shorter than a tile's keys), and tiles
 * cut by a range boundary are merged by log-sum-exp as in the other schedules.  The call then
 * occupies at most cu_budget CUs and leaves the rest free for work launched on another stream.
 *
 *   cu_budget   0: the whole device (exactly mtd_attn_prefill_chunk);  > 0: needs the workspace
 *               (else MTD_ERR_WORKSPACE);  < 0: MTD_ERR_INVALID_ARG
 * Every other argument, result and error is that of mtd_attn_prefill_chunk; results are correct
 * for every budget (their bits differ between schedules).
 */
int mtd_attn_prefill_chunk_cus(const mtd_kv_layer_t* kv, const void* q, int32_t chunk_len,
                               int32_t prefix_len, const int32_t* block_table, int32_t block_table_len,
                               int32_t num_q_heads, float scale, void* workspace, size_t workspace_bytes,
                               int32_t cu_budget, float* out, float* lse, void* stream);

/*
 * mtd_attn_prefill_workspace_bytes - size of the optional mtd_attn_prefill_chunk workspace:
 * chunk_len * num_q_heads * (head_dim + 1) * 4 bytes (the second halves' partial outputs and
 * log-sum-exps).  Returns 0 for arguments mtd_attn_prefill_chunk would reject.
 */
size_t mtd_attn_prefill_workspace_bytes(int32_t chunk_len, int32_t num_q_heads, int32_t head_dim);

/*
 * mtd_attn_decode_workspace_bytes - device workspace mtd_attn_decode needs for a batch whose
 * longest request holds at most max_kv_len tokens.  Returns 0 for arguments mtd_attn_decode would
 * reject.  The size is batch * P(max_kv_len) * num_q_heads * (head_dim + 1) * 4 bytes (split-K
 * partial outputs and log-sum-exps): a request of L tokens is split into runs of 64 tokens if
 * L <= 1024, 128 if L <= 2048, 256 if L <= 4096 and 512 above, and P(M) is the most runs any
 * L <= M can have (ceil(M / 64) up to 1024, 16 up to 8192, ceil(M / 512) above).
 */
size_t mtd_attn_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t max_kv_len,
                                       int32_t head_dim);

/*
 * mtd_attn_decode - one query token per request against that request's whole KV.
 *
 * Autoregressive decode emits one token per request per step over the request's whole cache, with
 * concurrent requests packed into one batch ("Optimizing ASR Models ...", sections ASR Model Primer
 * and Batched Inference; cookbook section Inference Pipeline, step 3).  The token of this step must
 * already be appended, and kv_lens counts it, so the query sits at position kv_lens[b] - 1 and sees
 * all kv_lens[b] keys.
 *
 *   q               bf16 [batch][num_q_heads][head_dim]
 *   kv_lens         int32 [batch], each in [1, max_kv_len]
 *   block_tables, bt_stride   int32 [batch][bt_stride], bt_stride >= ceil(max_kv_len / page_size)
 *                   (else MTD_ERR_CAPACITY)
 *   batch           >= 1;  max_kv_len: host upper bound of kv_lens, 1 .. MTD_MAX_CONTEXT
 *   num_q_heads     16;  scale > 0 and finite
 *   workspace       device scratch of at least mtd_attn_decode_workspace_bytes(batch, num_q_heads,
 *                   max_kv_len, head_dim) bytes, owned by the caller, contents ignored on entry and
 *                   unspecified on return; calls on different streams need different workspaces
 *   out             float32 [batch][num_q_heads][head_dim], written
 *   lse             float32 [batch][num_q_heads], written (natural log)
 *
 * The result of request b depends only on its own query, length and pages: it is bitwise the same
 * whatever the rest of the batch holds and wherever its pages sit in the pool.
 */
int mtd_attn_decode(const mtd_kv_layer_t* kv, const void* q, const int32_t* kv_lens,
                    const int32_t* block_tables, int32_t bt_stride, int32_t batch,
                    int32_t max_kv_len, int32_t num_q_heads, float scale, void* workspace,
                    size_t workspace_bytes, float* out, float* lse, void* stream);

/*
 * mtd_attn_decode_append - one decode step in one call: store each request's new K/V row, then
 * attend exactly as mtd_attn_decode does.
 *
 * Every autoregressive step adds the token it feeds to the KV cache and attends over the whole
 * cache including it ("Optimizing ASR Models ...", section ASR Model Primer, "Autoregressive
 * Decode").  At low concurrency that step is replayed from a captured graph (section Optimization
 * Strategies, AR Decode, "CUDA Graph"), and a replay pays for each launch it holds, so here the
 * store rides in the decode's split kernel: two launches per step instead of three.
 *
 *   k_new, v_new    bf16 [batch][num_kv_heads][head_dim] on the device, 16-byte aligned: the K and V
 *                   rows of each request's new token
 *   all other arguments as for mtd_attn_decode (kv_lens counts the new token)
 *
 * For kv_lens[b] in [1, max_kv_len], the pools and out / lse after the call are bit for bit those
 * of mtd_kv_append with one new row per request (cu_new = 0, 1, .., batch; start_pos[b] =
 * kv_lens[b] - 1; the same block tables) followed on the same stream by mtd_attn_decode with
 * these arguments.  A request whose kv_lens[b] lies outside that range stores nothing; a new token
 * whose page id is outside the pool is neither stored nor attended to, as with the two calls.
 * Errors: those of mtd_attn_decode, and MTD_ERR_INVALID_ARG when k_new or v_new is NULL or not
 * 16-byte aligned.
 */
int mtd_attn_decode_append(const mtd_kv_layer_t* kv, const void* q, const void* k_new, const void* v_new,
                           const int32_t* kv_lens, const int32_t* block_tables, int32_t bt_stride,
                           int32_t batch, int32_t max_kv_len, int32_t num_q_heads, float scale,
                           void* workspace, size_t workspace_bytes, float* out, float* lse, void* stream);

/* Bytes of the static device scratch mtd_attn_decode_noalloc uses on each GPU (64 MiB). */
#define MTD_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * mtd_attn_decode_noalloc - mtd_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  It allocates nothing and calls no allocating routine.
 *
 * Arguments, results and errors are those of mtd_attn_decode (same kernels, same bits), except:
 * the split partials go to a static device array of MTD_DECODE_NOALLOC_SCRATCH_BYTES per GPU
 * (mapped with the library, held until the process ends), so
 * mtd_attn_decode_workspace_bytes(batch, num_q_heads, max_kv_len, head_dim) must not exceed it,
 * else MTD_ERR_WORKSPACE (64 MiB holds 8128 partials: e.g. 64 requests of up to 64,512 tokens or
 * 31 of up to 131,072).  All calls on one GPU share that array and it keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other threads) race and give
 * unspecified results; order them on one stream.  The first call on a device looks up the array's
 * device address (hipGetSymbolAddress); a failure there returns MTD_ERR_HIP.
 */
int mtd_attn_decode_noalloc(const mtd_kv_layer_t* kv, const void* q, const int32_t* kv_lens,
                            const int32_t* block_tables, int32_t bt_stride, int32_t batch,
                            int32_t max_kv_len, int32_t num_q_heads, float scale, float* out,
                            float* lse, void* stream);

/*
 * mtd_qkv_proj - the QKV projection of new tokens: q = Wq x, k = Wk x, v = Wv x.
 *
 * Each decoder layer maps the hidden states (size 1024) of the tokens it processes to their
 * queries and their new keys and values ("Optimizing ASR Models ...", section ASR Model Primer,
 * component table: Qwen3, hidden 1024, GQA 16/8; cookbook section Model Architecture).  No bias.
 * The outputs have the layouts mtd_kv_append and the attention calls take.
 *
 *   x               bf16 [n_tok][hidden]
 *   w_qkv           bf16 [(num_q_heads + 2 num_kv_heads) * head_dim][hidden], the rows of Wq,
 *                   then Wk, then Wv ([out][in] layout: row n makes output feature n)
 *   n_tok           >= 0 (0 enqueues nothing);  hidden 1024;  num_q_heads 16;  num_kv_heads 8;
 *                   head_dim 128
 *   q               bf16 [n_tok][num_q_heads][head_dim], written: features 0 .. 2047
 *   k_new, v_new    bf16 [n_tok][num_kv_heads][head_dim], written: features 2048 .. 3071 and
 *                   3072 .. 4095
 * Feature f of a part is (head f / head_dim, dim f % head_dim).  Products are summed in float32
 * from bf16 operands and each result is rounded to bf16 (nearest, ties to even).  Every pointer
 * must be 16-byte aligned (else MTD_ERR_INVALID_ARG).  The result of a token does not depend on
 * n_tok or on the other tokens.
 */
int mtd_qkv_proj(const void* x, const void* w_qkv, int32_t n_tok, int32_t hidden,
                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, void* q, void* k_new,
                 void* v_new, void* stream);

/*
 * mtd_o_proj - the output projection of attention outputs: y = Wo o.
 *
 *   attn            float32 [n_tok][num_q_heads][head_dim], the attention output O (as written by
 *                   mtd_attn_prefill_chunk / mtd_attn_decode); rounded to bf16 (nearest, ties to
 *                   even), the decoder's activation type, before the product
 *   w_o             bf16 [hidden][num_q_heads * head_dim] ([out][in] layout; input feature
 *                   h * head_dim + d is head h, dim d)
 *   n_tok           >= 0 (0 enqueues nothing);  num_q_heads 16;  head_dim 128;  hidden 1024
 *   out             bf16 [n_tok][hidden], written (float32 sums rounded to bf16)
 * Every pointer must be 16-byte aligned (else MTD_ERR_INVALID_ARG).
 */
int mtd_o_proj(const float* attn, const void* w_o, int32_t n_tok, int32_t num_q_heads,
               int32_t head_dim, int32_t hidden, void* out, void* stream);

/* Most parts mtd_attn_merge combines in one call. */
#define MTD_MAX_MERGE_PARTS 1024

/*
 * mtd_attn_merge - combine attention results over disjoint key sets (log-sum-exp merge).
 *
 * The step after the gather when a request's KV is split by sequence over several GPUs: each GPU
 * runs mtd_attn_decode over its own page range (a block table starting at the range's first page
 * and kv_lens counting the range's tokens) and so produces that range's O and LSE; this call
 * combines the gathered partials into the result over all keys (the pages list multi-GPU support
 * for KV caches that outgrow one GPU as ongoing work: "Optimizing ASR Models ...", section What's
 * Next).  It is exact up to rounding: LSE = ln sum_k exp(lse_k), O = sum_k exp(lse_k - LSE) o_k.
 *
 *   o_parts     float32 [n_parts][n_rows][head_dim], part k's outputs (rows = tokens x heads)
 *   lse_parts   float32 [n_parts][n_rows], part k's natural-log LSE; -inf = no keys (zero weight)
 *   n_parts     1 .. MTD_MAX_MERGE_PARTS;  n_rows >= 0 (0 enqueues nothing);  head_dim 128
 *   out         float32 [n_rows][head_dim], written;  lse  float32 [n_rows], written
 * A row whose parts all have LSE = -inf gets O = 0 and LSE = -inf.  o_parts and out must be
 * 16-byte aligned (else MTD_ERR_INVALID_ARG).
 */
int mtd_attn_merge(const float* o_parts, const float* lse_parts, int32_t n_parts, int32_t n_rows,
                   int32_t head_dim, float* out, float* lse, void* stream);

/*
 * mtd_measure_page_read - measurement aid, not part of attention: read K/V page blocks the way
 * mtd_attn_decode reads them, and nothing else.
 *
 * Decode time is set by streaming a batch's K/V pages from HBM, so the figure to hold it against
 * is the rate this access pattern reaches on the device.  One wavefront per (pages_per_wave
 * consecutive entries of page_ids, KV head) reads the whole K and V blocks of those pages with the
 * decode's lane layout and 16-byte non-temporal loads, folds the words together and writes one
 * word per lane to sink.  Bytes read: 2 * num_kv_heads * page_size * head_dim * 2 per valid id.
 *
 *   page_ids        int32 [n_ids] on the device; ids outside [0, num_pages) are skipped
 *   n_ids           >= 1;  pages_per_wave 1 .. 64
 *   sink            uint32 [mtd_measure_page_read_sink_words(n_ids, pages_per_wave)], written
 *                   (the folded words, meaningful only as a dependency of the loads)
 */
int mtd_measure_page_read(const mtd_kv_layer_t* kv, const int32_t* page_ids, int32_t n_ids,
                          int32_t pages_per_wave, uint32_t* sink, size_t sink_words, void* stream);

/* Words mtd_measure_page_read writes to sink; 0 for arguments it would reject. */
size_t mtd_measure_page_read_sink_words(int32_t n_ids, int32_t pages_per_wave);

/* Static description of a status code (never NULL). */
const char* mtd_status_string(int status);

/* Detail of the last failed call on the calling thread ("" if none).  Valid until the next call. */
const char* mtd_last_error(void);

/* MTD_ABI_VERSION of the built library. */
int mtd_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MTD_H */
