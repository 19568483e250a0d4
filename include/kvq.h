/*
 * kvq.h -- quantized KV-cache store and compressed-domain attention on MI355X (gfx950).
 *
 * C ABI of libkvq.so.  Every pointer argument marked "device" is device memory
 * owned by the caller; the library never allocates, frees or synchronises.
 * Every call is asynchronous on the HIP stream passed as `stream` (a
 * hipStream_t; NULL is the default stream).  Arguments are validated on the
 * host before anything is enqueued: on error nothing is launched and the
 * status says why (kvq_last_error() gives a message for the calling thread).
 * A launch failure maps to KVQ_ERR_HIP.  Device-side values (slots, positions,
 * lengths, page tables) must be consistent with the shapes passed: the
 * kernels trust them to stay inside the planes.
 *
 * Sources (cited by page title and section):
 *   [tract-RFC]     "Heads-up / RFC: int4 + Hadamard KV-cache quantization
 *                   (CPU + Metal)", tract discussion #2402
 *   [FreeToken-268] "feat(kvcache): sub-byte Q4_0 and Q6_0 KV cache
 *                   quantization", FreeToken PR #268
 *   [Open-TQ-Metal] "Open-TQ-Metal: Fused Compressed-Domain Attention for
 *                   Long-Context LLM Inference on Apple Silicon", arXiv 2604.16957
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Cache encodings.  4-bit codes of element j are packed two per byte, element
 * 2j in the low nibble ([FreeToken-268] Storage layouts); rows are per token,
 * per kv head, separately for K and V.
 *   HAD_INT4  [tract-RFC] What's done (CPU); Architecture > Data flow (decode):
 *             row rotated by the orthonormal Hadamard (fast transform), then
 *             per-token symmetric int4 in [-8, 7], scale amax/8 as one f32.
 *             payload D/2 bytes, record 4 bytes.  D must be a power of two.
 *   Q4_0      [FreeToken-268] Summary, Storage layouts: 32-element blocks,
 *             fp16 scale amax/8, codes [-8, 7].  payload D/2, record 2*D/32.
 *   Q6_0      [FreeToken-268] Storage layouts: per block 16-byte low-nibble
 *             plane then 8-byte plane of the top two bits (value 4k+i at byte k,
 *             bits 2i), fp16 scale amax/32, codes [-32, 31].
 *             payload 24*D/32, record 2*D/32.
 *   ASYM_INT4_G32 [Open-TQ-Metal] Background (per-group asymmetric int4):
 *             groups of 32, min-max affine map, fp16 scale (max-min)/15 then
 *             fp16 zero (= min) per group, unsigned codes [0, 15].
 *             payload D/2, record 4*D/32.
 *   Q8_0      [FreeToken-268] Summary and memory table (8-bit block scheme,
 *             1.0625 bytes per element): 32-element blocks, fp16 scale amax/128,
 *             codes [-128, 127] stored one per byte as two's complement, in
 *             element order.  payload D, record 2*D/32.
 * Range.  The attention kernels run the P V product on fp16 operands.  For the
 * layouts with fp16 scales (Q4_0, Q6_0, ASYM_INT4_G32, Q8_0) each dequantised V
 * element is formed in fp16, so V rows must dequantise to within +-65504 (a
 * row past that reads as infinite).  HAD_INT4 folds its f32 V scale into the
 * softmax weights relative to a power of two (no limit short of f32's). */
typedef enum kvq_layout {
  KVQ_LAYOUT_HAD_INT4 = 0,
  KVQ_LAYOUT_Q4_0 = 1,
  KVQ_LAYOUT_Q6_0 = 2,
  KVQ_LAYOUT_ASYM_INT4_G32 = 3,
  KVQ_LAYOUT_Q8_0 = 4
} kvq_layout;

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = 1, /* null pointer, bad size, inconsistent shapes     */
  KVQ_ERR_UNSUPPORTED = 2, /* (layout, head_dim, gqa) not built into the library */
  KVQ_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required         */
  KVQ_ERR_HIP = 4          /* a HIP launch failed                                */
} kvq_status;

/* Flags of kvq_attend_prefill_causal. */
#define KVQ_PREFILL_NO_CAUSAL_SKIP 1u /* visit KV tiles wholly past the causal limit too */

/* The paged cache.  All planes are device memory owned by the caller; the
 * library reads and writes them only inside calls.
 *   k_payload, v_payload  uint8 [num_pages][num_kv_heads][page_size][payload_bytes]
 *   k_scale,   v_scale    uint8 [num_pages][num_kv_heads][page_size][scale_bytes]
 *   k_recent,  v_recent   f32   [max_batch][num_kv_heads][n_recent][head_dim]
 * The recent window ([tract-RFC] Causality & mixed precision, n_recent) keeps
 * the newest n_recent positions of each batch row as exact f32 rows (rotated
 * for HAD_INT4) in a ring indexed by position % n_recent; may be NULL when
 * n_recent == 0.  page_size is a power of two >= 16; head_dim is 128 or 256;
 * num_pages * page_size is at most INT32_MAX (slots are int32), while byte
 * offsets into the planes are 64-bit, so a plane may exceed 4 GiB. */
typedef struct kvq_cache {
  int32_t layout;       /* kvq_layout */
  int32_t head_dim;
  int32_t num_kv_heads;
  int32_t page_size;
  int32_t num_pages;
  int32_t n_recent;
  int32_t max_batch;
  int32_t reserved;     /* must be 0 */
  void* k_payload;
  void* v_payload;
  void* k_scale;
  void* v_scale;
  float* k_recent;
  float* v_recent;
} kvq_cache;

/* Bytes of one stored row (per token, per kv head, per tensor); 0 if the
 * (layout, head_dim) pair is not supported. */
size_t kvq_payload_bytes(int32_t layout, int32_t head_dim);
size_t kvq_scale_bytes(int32_t layout, int32_t head_dim);

/* Quantize-on-append.  [tract-RFC] Architecture > Data flow (decode), append
 * step, and the on-device append kernel asked for under Metal integration;
 * [FreeToken-268] Changes (store kernel); encodings as documented above.
 *   k_new, v_new  device f32 [n_tok][num_kv_heads][head_dim]
 *   slot          device int32 [n_tok]: physical page * page_size + offset
 *   batch_idx     device int32 [n_tok]: batch row (window ring row)
 *   pos           device int32 [n_tok]: absolute position of the token
 *   seq_len       device int32 [max_batch]: row length after this store
 * Every token is quantised into its slot.  When n_recent > 0 a token whose
 * pos >= seq_len[row] - n_recent is also written as an f32 row into the ring
 * slot pos % n_recent (so a multi-token append never writes one ring slot
 * twice).  n_tok == 0 is a no-op.  Codes and scales are bit-exact functions of
 * the inputs (ties to even, f32 division, fp16 fields saturate at 65504). */
kvq_status kvq_store(const kvq_cache* cache, const float* k_new, const float* v_new,
                     int32_t n_tok, const int32_t* slot, const int32_t* batch_idx,
                     const int32_t* pos, const int32_t* seq_len, void* stream);

/* The same quantize-on-append for a chunk of n_q tokens of every batch row,
 * with the slots taken from the block table: token i of row b goes to position
 * q_start[b] + i, and the row's length after the append is q_start[b] + n_q
 * (which decides the window rows, as in kvq_store).
 *   k_new, v_new  device f32 [batch][n_q][num_kv_heads][head_dim]
 *   q_start       device int32 [batch]: cached tokens of each row before the chunk
 *   block_table   device int32 [batch][max_pages_per_seq]
 *   max_seq_len   host bound on q_start[b] + n_q; max_pages_per_seq * page_size
 *                 must cover it (a position the table does not cover is skipped)
 * batch must not exceed max_batch when n_recent > 0.  n_q == 0 is a no-op. */
kvq_status kvq_store_chunk(const kvq_cache* cache, const float* k_new, const float* v_new,
                           int32_t batch, int32_t n_q, const int32_t* q_start,
                           const int32_t* block_table, int32_t max_pages_per_seq,
                           int32_t max_seq_len, void* stream);

/* The split-K work split kvq_attend_decode executes for these arguments (it
 * depends on the shape and the device's compute-unit count): each wave
 * streams *wave_tokens consecutive tokens of one (batch row, kv head) as one
 * run (whole chunk_tokens chunks, or a half or quarter chunk for short
 * contexts), and a block merges its four waves' runs into one partial of
 * *partial_tokens tokens, which the reduce then merges.  Every level is the
 * same online-softmax merge of the chunk partials of [Open-TQ-Metal]'s split-K
 * paragraphs, so the result matches chunks of chunk_tokens up to float
 * re-association.  Errors as for kvq_attend_decode's argument checks. */
kvq_status kvq_decode_split(const kvq_cache* cache, int32_t batch, int32_t num_q_heads,
                            int32_t max_seq_len, int32_t chunk_tokens, int32_t* wave_tokens,
                            int32_t* partial_tokens);

/* The same for rows of the given lengths (host int32 [batch], each in
 * [0, max_seq_len]).  When even runs of four chunks leave a batch of several
 * rows more blocks than the device holds at once, the decode kernels choose the
 * run length per call from seq_len, among 4, 2 and 1.5 chunks, as the one
 * with the fewest whole rounds of resident blocks times a wave's time (a
 * start-up of about four 32-token steps plus its run); a ragged batch can then
 * take shorter runs that fill its last round.  kvq_decode_split reports that
 * choice for rows of max_seq_len tokens, this call for these lengths (the
 * int8-query kernels; the float-query kernels hold fewer blocks per CU). */
kvq_status kvq_decode_split_lengths(const kvq_cache* cache, int32_t batch, int32_t num_q_heads,
                                    const int32_t* seq_len_host, int32_t max_seq_len,
                                    int32_t chunk_tokens, int32_t* wave_tokens,
                                    int32_t* partial_tokens);

/* Workspace of kvq_attend_decode: room for split-K partials (o_c, m_c, l_c) per
 * (batch, query head, chunk), plus the window partial.  (The decode kernel
 * prepares its int8 queries itself.)  Returns 0 for invalid arguments. */
size_t kvq_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_seq_len, int32_t chunk_tokens);

/* Fused compressed-domain decode attention, one query per batch row.
 * [Open-TQ-Metal] Algorithm 1 and the split-K paragraphs: the packed cache is
 * read directly (no dequantised S x d temporary), the sequence is split into
 * chunks of chunk_tokens tokens that run in parallel, each emitting
 * (o_c, m_c, l_c), and a reduce merges them with the online-softmax
 * correction.  Scores are int8(Q) . int4/int6(K) -> i32 per block with the
 * scales applied outside ([tract-RFC] Architecture > Data flow (decode)); GQA
 * maps query head h to kv head h / (num_q_heads / num_kv_heads)
 * ([Open-TQ-Metal] SIMD and threadgroup organization).  For HAD_INT4 the query
 * is rotated first and the output rotated back.
 *   q            device f32 [batch][num_q_heads][head_dim]
 *   out          device f32 [batch][num_q_heads][head_dim]
 *   block_table  device int32 [batch][max_pages_per_seq]: physical page of each
 *                logical page of the row
 *   seq_len      device int32 [batch]: cached tokens of each row (<= max_seq_len);
 *                the newest min(seq_len, n_recent) are read from the window
 *   max_seq_len  host bound on seq_len (sizes the grid)
 *   chunk_tokens split-K chunk, a multiple of 128
 * num_q_heads must be a multiple of num_kv_heads.  A row with
 * seq_len 0 gets zeros.  alpha is the score scale (1/sqrt(d), or 1.0 for
 * RMS-normalised Q/K, [Open-TQ-Metal] Section 4). */
kvq_status kvq_attend_decode(const kvq_cache* cache, const float* q, float* out,
                             int32_t batch, int32_t num_q_heads, float alpha,
                             const int32_t* block_table, int32_t max_pages_per_seq,
                             const int32_t* seq_len, int32_t max_seq_len,
                             int32_t chunk_tokens, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Decode in the float-query mode: the quantised tokens are scored with the f32
 * query (rotated for HAD_INT4) instead of its int8 form, the way
 * [FreeToken-268] Changes (the attention kernel's K/V load unpacks the codes
 * into a standard attention) and [Open-TQ-Metal]'s fused kernel (a
 * pre-divided floating-point query against the packed nibbles) read the
 * cache.  The integer dots run on the same packed codes with the query
 * expanded to three int8 terms, sq * (q8 + r1 / 254 + r2 / 254^2) with
 * sq = amax|q| / 127, which holds the f32 query to within about amax|q| / 2^24
 * per element (the resolution of f32 at the vector's largest element); V, the
 * window, the merge and every argument are those of kvq_attend_decode (same
 * workspace size and errors). */
kvq_status kvq_attend_decode_float_q(const kvq_cache* cache, const float* q, float* out,
                                     int32_t batch, int32_t num_q_heads, float alpha,
                                     const int32_t* block_table, int32_t max_pages_per_seq,
                                     const int32_t* seq_len, int32_t max_seq_len,
                                     int32_t chunk_tokens, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* kvq_attend_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same kernels, with the split-K partials in a device scratch array of
 * the library instead of a caller's workspace.  Every argument and result is
 * that of kvq_attend_decode (int8-query mode).  No memory is allocated or
 * freed, by the library or any routine it calls; each device holds one
 * scratch array of KVQ_DECODE_NOALLOC_SCRATCH_BYTES from the library's load
 * until the process ends.  A call needs batch * num_q_heads * (head_dim + 4)
 * * 4 bytes per split-K group of the call (plus one group for the window);
 * a call needing more than the scratch returns KVQ_ERR_WORKSPACE and launches
 * nothing.  Calls on one device share its array: calls that overlap on that
 * device (concurrent streams or host threads) race and give wrong results,
 * so the caller orders them (one stream, or events).  Stream-ordered calls
 * are independent: each overwrites every partial its own reduce reads.  The
 * calling thread's current device must be the stream's device. */
#define KVQ_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
kvq_status kvq_attend_decode_noalloc(const kvq_cache* cache, const float* q, float* out,
                                     int32_t batch, int32_t num_q_heads, float alpha,
                                     const int32_t* block_table, int32_t max_pages_per_seq,
                                     const int32_t* seq_len, int32_t max_seq_len,
                                     int32_t chunk_tokens, void* stream);

/* The two phases of kvq_attend_decode as separate calls, for callers that time
 * or schedule them apart ([Open-TQ-Metal] split-K paragraphs: a partial phase
 * and a reduce phase ordered by their data dependency; here by stream order).
 * kvq_attend_decode_partial computes a partial per chunk, merges each group of
 * four consecutive chunks' partials at once (the first level of the same
 * online-softmax merge) and writes one partial per group (and the window
 * partial) into the workspace; kvq_attend_decode_reduce merges those into out.
 * Arguments mean what they mean for kvq_attend_decode and must be identical
 * between the two calls. */
kvq_status kvq_attend_decode_partial(const kvq_cache* cache, const float* q, int32_t batch,
                                     int32_t num_q_heads, float alpha, const int32_t* block_table,
                                     int32_t max_pages_per_seq, const int32_t* seq_len,
                                     int32_t max_seq_len, int32_t chunk_tokens, void* workspace,
                                     size_t workspace_bytes, void* stream);
kvq_status kvq_attend_decode_reduce(const kvq_cache* cache, float* out, int32_t batch,
                                    int32_t num_q_heads, const int32_t* seq_len, int32_t max_seq_len,
                                    int32_t chunk_tokens, const void* workspace, size_t workspace_bytes,
                                    void* stream);

/* Workspace of kvq_attend_prefill_causal and kvq_prefill_full_then_store:
 * split-K partials (o_c as head_dim f16 values with a power-of-two scale,
 * m_c, l_c; 2 head_dim + 16 bytes) per (batch, query, query head, chunk of
 * the shortest split, 512 tokens; the call picks chunks of at least that
 * length), plus the window partial, then the prepared queries per (batch,
 * query, query head), then room for the chunk's rotated K and V rows (the
 * full-precision prefill of HAD_INT4).  Returns 0 for invalid arguments. */
size_t kvq_prefill_workspace_bytes(int32_t batch, int32_t n_q, int32_t num_q_heads,
                                   int32_t head_dim, int32_t max_seq_len);

/* Causal prefill over the packed cache, called after kvq_store of the chunk.
 * [tract-RFC] Architecture (the prefill path: store the chunk first, then run
 * attention in which every query is bounded by its own position) and
 * Causality & mixed precision (skipping the work past a query's bound gives
 * the same bits as computing it and masking).  Query i of row b sits at
 * position q_start[b] + i and, when causal != 0, sees tokens t <= q_start[b] + i;
 * KV tiles wholly past the limit are skipped unless flags has
 * KVQ_PREFILL_NO_CAUSAL_SKIP (same bits, masked tiles streamed).  The window
 * is the last n_recent positions of the row, the same for every query, masked
 * per query like the packed tokens.  Scores, scales and the HAD_INT4 rotation
 * are those of kvq_attend_decode; a query whose limit covers the whole row
 * gets the decode output up to float re-association (the two kernels add the
 * same terms in different orders; tested to 2e-3 * max|o|).
 *   q          device f32 [batch][n_q][num_q_heads][head_dim]
 *   out        device f32 [batch][n_q][num_q_heads][head_dim]
 *   causal     0 or 1; with 0 every query sees all seq_len[b] tokens
 *   q_start    device int32 [batch] (may be NULL when causal == 0); the limits
 *              are meaningful for q_start[b] + n_q <= seq_len[b]; a query
 *              that sees no token gets zeros
 *   workspace  at least kvq_prefill_workspace_bytes(...) bytes of device memory
 * Other arguments as for kvq_attend_decode.  Errors: KVQ_ERR_INVALID_ARG for
 * null pointers, n_q < 1, causal not 0/1 or unknown flags;
 * KVQ_ERR_WORKSPACE when the workspace is too small; nothing is launched then. */
kvq_status kvq_attend_prefill_causal(const kvq_cache* cache, const float* q, float* out,
                                     int32_t batch, int32_t n_q, int32_t num_q_heads,
                                     float alpha, int32_t causal, const int32_t* q_start,
                                     const int32_t* block_table, int32_t max_pages_per_seq,
                                     const int32_t* seq_len, int32_t max_seq_len, uint32_t flags,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* Full-precision prefill, then quantise-on-store.  [Open-TQ-Metal]
 * prefill/decode selection paragraph: a multi-query step attends over the
 * full-precision K, V and only then quantises them into the cache, while decode
 * reads the packed cache.  Query i of row b (position q_start[b] + i) attends
 * over the row's cached prefix, read as the cache holds it before this call
 * (packed tokens, and the window's f32 rows for its newest min(q_start[b],
 * n_recent) positions), and over the chunk's own tokens as the exact f32 rows
 * k_new, v_new (rotated for HAD_INT4, like window rows), with the causal limit
 * q_start[b] + i when causal != 0.  Then the chunk is stored as by
 * kvq_store_chunk.  The prefix's scores, the window and the merge are those of
 * kvq_attend_prefill_causal with seq_len = q_start.
 *   q             device f32 [batch][n_q][num_q_heads][head_dim]
 *   k_new, v_new  device f32 [batch][n_q][num_kv_heads][head_dim]
 *   out           device f32 [batch][n_q][num_q_heads][head_dim]
 *   q_start       device int32 [batch]: cached tokens of each row before the chunk
 *   max_seq_len   host bound on q_start[b] + n_q
 *   workspace     kvq_prefill_workspace_bytes(batch, n_q, num_q_heads, head_dim,
 *                 max_seq_len) bytes of device memory
 * Errors as for kvq_attend_prefill_causal and kvq_store_chunk; nothing is
 * launched on an error. */
kvq_status kvq_prefill_full_then_store(const kvq_cache* cache, const float* q, const float* k_new,
                                       const float* v_new, float* out, int32_t batch, int32_t n_q,
                                       int32_t num_q_heads, float alpha, int32_t causal,
                                       const int32_t* q_start, const int32_t* block_table,
                                       int32_t max_pages_per_seq, int32_t max_seq_len,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Read-only streaming probe (measurement, not part of the method): reads n
 * (1..4) device buffers src[i] of bytes[i] bytes (host arrays) once, in one
 * launch across the whole device, with the direct-to-LDS 16-byte nontemporal
 * loads the decode kernel streams with (the data lands in LDS that nothing
 * reads).  Buffers and sizes must be 16-byte aligned.  The bench times it over
 * a layer's four planes: the attainable HBM read rate for those bytes, which
 * the decode kernel's rate is compared with. */
kvq_status kvq_debug_stream_read(int32_t n, const void* const* src, const size_t* bytes, void* stream);

/* Test exports for the bit-exact gates. */

/* Query preparation of the attention kernels: rotation (HAD_INT4 only) and
 * per-vector int8, sq = amax/127 ([tract-RFC] data flow, int8(Q_rot)).
 *   q device f32 [n_vec][head_dim]; q8 device int8 [n_vec][head_dim]; sq device f32 [n_vec] */
kvq_status kvq_debug_quantize_q(int32_t layout, const float* q, int32_t n_vec, int32_t head_dim,
                                int8_t* q8, float* sq, void* stream);

/* The decode kernel's per-block integer scores I[t][g] = sum_j q8_j * code_tj
 * over block g (the whole row for HAD_INT4), for quantised tokens
 * t < seq_len[b] - n_recent; other entries are left untouched.
 *   scores     device int32 [batch][num_q_heads][max_seq_len][n_groups],
 *              n_groups = 1 for HAD_INT4, head_dim/32 otherwise
 *   workspace  kvq_decode_workspace_bytes(batch, num_q_heads, head_dim,
 *              max_seq_len, 512) bytes of device memory (the prepared queries) */
kvq_status kvq_debug_qk_i32(const kvq_cache* cache, const float* q, int32_t batch,
                            int32_t num_q_heads, const int32_t* block_table,
                            int32_t max_pages_per_seq, const int32_t* seq_len,
                            int32_t max_seq_len, int32_t* scores, void* workspace,
                            size_t workspace_bytes, void* stream);

const char* kvq_status_string(kvq_status status);
const char* kvq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
