/*
 * attn.h — causal multi-head / grouped-query attention for MI355X (gfx950).
 *
 * Eight operations, all hand-written HIP kernels behind a plain C ABI:
 *
 *  - attn_prefill: causal self-attention of T queries over the same T keys,
 *    computed block by block with an online softmax so that the T x T score
 *    matrix never exists in memory (the blockwise softmax-statistics method
 *    of the llm-from-scratch "Project Overview" page, "Performance Layer:
 *    kernel/ and parallel/"; causal MHA/GQA as in the microLLM-rocm README,
 *    "Why this project exists").
 *
 *  - attn_decode_paged: one new query token per sequence attending over that
 *    sequence's cached keys and values, which live in fixed-size pages of a
 *    shared pool addressed through a per-sequence block table (the paged KV
 *    cache of the RoseLLM README, "What is inside" and "Systems highlights",
 *    "Inference and serving"; KV-cache decode with BF16 storage and FP32
 *    accumulation as in the microLLM-rocm README, "Why this project exists").
 *    It runs as a split-KV kernel writing partial results, followed by a
 *    log-sum-exp combine kernel.
 *
 *  - attn_prefill_paged: chunked prefill over the paged cache: the last Tq
 *    tokens of each sequence (a chunk processed after the sequence's prefix
 *    was cached, as in the chunked prefill and prefix reuse of the RoseLLM
 *    README, "Systems highlights", "Inference and serving") attend over all
 *    of the sequence's cached keys, causally.  It is the prefill kernel
 *    reading its key/value tiles page by page through the block table.
 *
 *  - attn_decode_paged_fp8: the same decode over a cache whose keys and
 *    values are stored as FP8 E4M3 with one scale per tensor (the FP8 KV
 *    cache of the microLLM-rocm README, "Why this project exists").
 *
 *  - attn_prefill_varlen: causal prefill of a ragged batch, sequences of
 *    different lengths packed token after token (ragged / varlen prefill,
 *    RoseLLM README, "Systems highlights", "Inference and serving"); each
 *    sequence is an independent causal prefill.
 *
 *  - attn_kv_append: writes the newest tokens' keys and values into their
 *    slots of the paged cache (the KV-cache writer of the RoseLLM README,
 *    "Systems highlights", "Inference and serving"), the step before decode
 *    or chunked prefill reads them.
 *
 *  - attn_prefill_paged_append: KV append and chunked prefill in one launch
 *    (the fused KV append of the RoseLLM README, "Systems highlights",
 *    "Inference and serving", with its chunked prefill): the chunk's keys
 *    and values arrive as dense tensors, the attention reads them from there
 *    (and the older keys from the pages), and the same launch writes them
 *    into their page slots.  Same results as attn_kv_append followed by
 *    attn_prefill_paged, bit for bit.
 *
 *  - attn_decode_paged_append: the one-token KV append fused into the paged
 *    decode (the same README passage, with its paged decode): the newest
 *    token is read from dense tensors and written into its slot by the
 *    combine kernel; bit for bit attn_kv_append followed by
 *    attn_decode_paged.
 *
 * What is computed.  For query head h, the kv head read is h / (Hq / Hkv)
 * (consecutive groups of query heads share one kv head).  For a query q and
 * its visible keys k_j with values v_j:
 *     s_j = scale * <q, k_j>,   out = sum_j softmax(s)_j v_j,
 *     lse = ln sum_j exp(s_j)   (natural log, scale included).
 * Prefill: query t sees keys 0..t (inclusive).  Decode: the query of
 * sequence b stands at position seq_lens[b]-1 and sees keys
 * 0..seq_lens[b]-1, so its own key and value must already be in the cache.
 * Chunked prefill: query t of sequence b stands at position
 * seq_lens[b] - Tq + t and sees keys 0..seq_lens[b] - Tq + t (the chunk's
 * own keys and values must already be in the cache).
 *
 * Conventions for every entry point.
 *  - Pointers marked "device" are device memory owned by the caller; the
 *    library never allocates, frees, reads on the host or synchronises.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and runs asynchronously; the call returns once it is enqueued.
 *  - The return value is an attn_status_t.  Every argument check runs before
 *    any HIP call, so a rejected call touches no device state.  A failed
 *    launch returns ATTN_ERR_HIP; attn_last_error_message() describes the
 *    most recent failure on the calling thread.
 *  - Tensors are dense, row-major, in the layouts given below; 16-byte
 *    aligned base pointers are required for q, k, v, out, the page pools and
 *    the workspace, 4-byte alignment for lse, block_table and seq_lens.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = -1, /* null pointer, bad size, misaligned, Hq % Hkv != 0, ... */
    ATTN_ERR_UNSUPPORTED = -2, /* valid request this build has no kernel for (dtype, d, page size, group) */
    ATTN_ERR_WORKSPACE = -3,   /* workspace null or smaller than attn_decode_workspace_bytes() */
    ATTN_ERR_HIP = -4          /* the HIP runtime reported an error while enqueuing */
} attn_status_t;

/* Element types.  Entry points take the value as a plain int `dtype`, so
 * that any other value is a defined input (rejected with
 * ATTN_ERR_INVALID_ARG) rather than an out-of-range enum. */
typedef enum attn_dtype {
    ATTN_F32 = 0,  /* float32 q/k/v/out; fp32 arithmetic throughout */
    ATTN_BF16 = 1  /* bfloat16 q/k/v/out; fp32 accumulation, bf16 MFMA products */
} attn_dtype_t;

/*
 * Causal prefill (blockwise online softmax; see the file header).
 *
 *   q, out : device, [B, Hq,  T, d] in `dtype`
 *   k, v   : device, [B, Hkv, T, d] in `dtype`
 *   lse    : device, [B, Hq, T] float32, or NULL to skip it
 *   B, T   : >= 0 (B == 0 or T == 0 enqueues nothing and returns ATTN_OK)
 *   Hq,Hkv : >= 1, Hq % Hkv == 0
 *   d      : 64 or 128
 *   scale  : multiplies q.k (usually 1/sqrt(d)); any finite value
 *   dtype  : ATTN_BF16 (d 64 or 128) or ATTN_F32 (d 64 or 128)
 * out is written with round-to-nearest-even from the fp32 accumulator.
 * q, k, v must hold finite values.
 */
int attn_prefill(const void* q, const void* k, const void* v, void* out, float* lse,
                 int B, int Hq, int Hkv, int T, int d, float scale,
                 int dtype, hipStream_t stream);

/*
 * Chunked causal prefill over a paged KV cache (see the file header).
 *
 *   q, out         : device, [B, Hq, Tq, d] in `dtype`; row t of sequence b
 *                    is the query at position seq_lens[b] - Tq + t
 *   k_pages,v_pages: device, [num_pages, Hkv, page_size, d] in `dtype`, as
 *                    for attn_decode_paged
 *   block_table    : device int32 [B, max_pages_per_seq], as for decode;
 *                    entries past ceil(seq_lens[b] / page_size) are never read
 *   seq_lens       : device int32 [B]; cached tokens per sequence, the chunk
 *                    included: each in [Tq, max_pages_per_seq * page_size]
 *   lse            : device float32 [B, Hq, Tq], or NULL to skip it
 *   B, Tq          : >= 0 (either 0 enqueues nothing and returns ATTN_OK)
 *   Hq, Hkv        : >= 1, Hq % Hkv == 0, Hq / Hkv <= 128
 *   dtype          : ATTN_BF16; d = 128 or 64; page_size = 16;
 *                    max_pages_per_seq <= 8192 (contexts up to 131072 tokens)
 * out is written with round-to-nearest-even from the fp32 accumulator; q and
 * the cached tokens must hold finite values, other slots may hold anything.
 * The block table and seq_lens are read on the device only; values outside
 * the ranges above are undefined behaviour (check them with
 * attn_validate_chunk_metadata).  No workspace is needed.
 */
int attn_prefill_paged(const void* q, const void* k_pages, const void* v_pages,
                       const int32_t* block_table, const int32_t* seq_lens,
                       void* out, float* lse,
                       int B, int Hq, int Hkv, int Tq, int d, int page_size, int num_pages,
                       int max_pages_per_seq, float scale, int dtype,
                       hipStream_t stream);

/*
 * Causal prefill of a ragged batch packed along the token axis.
 *
 *   q, out     : device, [total_tokens, Hq, d] in `dtype`
 *   k, v       : device, [total_tokens, Hkv, d] in `dtype`
 *   lse        : device, [total_tokens, Hq] float32, or NULL to skip it
 *   cu_seqlens : device int32 [num_seqs + 1]: sequence s holds tokens
 *                cu_seqlens[s] .. cu_seqlens[s+1]-1; cu_seqlens[0] = 0, the
 *                entries do not decrease, cu_seqlens[num_seqs] = total_tokens
 *   max_seqlen : >= every sequence's length (sizes the launch)
 *   Hq, Hkv    : >= 1, Hq % Hkv == 0, Hq / Hkv <= 128
 *   dtype      : ATTN_BF16; d = 128 or 64
 * Token i of sequence s sees keys cu_seqlens[s] .. cu_seqlens[s] + i.
 * num_seqs, total_tokens or max_seqlen equal to 0 enqueues nothing.
 * cu_seqlens is read on the device only; values outside the contract above
 * are undefined behaviour (check them with attn_validate_varlen_metadata).
 * q, k, v must hold finite values.
 */
int attn_prefill_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                        const int32_t* cu_seqlens, int num_seqs, int total_tokens, int max_seqlen,
                        int Hq, int Hkv, int d, float scale, int dtype, hipStream_t stream);

/*
 * Host-side check of a host copy of cu_seqlens against the contract of
 * attn_prefill_varlen.  Returns ATTN_OK or ATTN_ERR_INVALID_ARG.
 */
int attn_validate_varlen_metadata(const int32_t* cu_seqlens_host, int num_seqs, int total_tokens,
                                  int max_seqlen);

/*
 * KV append: copy the last Tn tokens' keys and values of each sequence into
 * the paged cache.
 *
 *   k_new, v_new   : device, [B, Hkv, Tn, d] in `dtype`; token t of sequence
 *                    b goes to position seq_lens[b] - Tn + t
 *   k_pages,v_pages: device, [num_pages, Hkv, page_size, d] in `dtype`; only
 *                    the B * Tn written (page, slot) rows change, every kv head
 *   block_table    : device int32 [B, max_pages_per_seq], as for decode
 *   seq_lens       : device int32 [B]; each sequence's length after the
 *                    append, in [Tn, max_pages_per_seq * page_size] (the same
 *                    array then serves attn_decode_paged or attn_prefill_paged)
 *   dtype          : ATTN_BF16; d = 128 or 64; page_size = 16
 * Values are copied bit for bit.  Two appended tokens must not name the same
 * (page, slot); the block table and seq_lens are read on the device only
 * (check them with attn_validate_chunk_metadata, chunk_len = Tn).
 */
int attn_kv_append(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                   const int32_t* block_table, const int32_t* seq_lens,
                   int B, int Hkv, int Tn, int d, int page_size, int num_pages,
                   int max_pages_per_seq, int dtype, hipStream_t stream);

/*
 * Fused KV append + chunked prefill: the work of attn_kv_append(k_new, v_new,
 * k_pages, v_pages, ...) followed by attn_prefill_paged(q, k_pages, v_pages,
 * ...) with the same sizes, in one launch; out, lse and the pools come out
 * bit for bit as from those two calls.
 *
 *   q, out         : device, [B, Hq, Tq, d]; row t of sequence b is the query
 *                    at position seq_lens[b] - Tq + t
 *   k_new, v_new   : device, [B, Hkv, Tq, d]: the chunk's keys and values,
 *                    token t at position seq_lens[b] - Tq + t
 *   k_pages,v_pages: device, [num_pages, Hkv, page_size, d]; read for the
 *                    positions below seq_lens[b] - Tq, written (bit-exact
 *                    copies of k_new / v_new) at the chunk's positions; no
 *                    other byte changes
 *   block_table    : device int32 [B, max_pages_per_seq], as for decode
 *   seq_lens       : device int32 [B]; lengths after the append, each in
 *                    [Tq, max_pages_per_seq * page_size]
 *   lse            : device float32 [B, Hq, Tq], or NULL to skip it
 *   B, Tq          : >= 0 (either 0 enqueues nothing and returns ATTN_OK)
 *   Hq, Hkv        : >= 1, Hq % Hkv == 0, Hq / Hkv <= 128
 *   dtype          : ATTN_BF16; d = 128 or 64; page_size = 16;
 *                    max_pages_per_seq <= 8192
 * Within the launch no (page, slot) is both written and read: the chunk's
 * keys are read from k_new / v_new only.  So, beyond the conditions of the
 * two calls it replaces (two chunk tokens must not name the same (page,
 * slot)), a slot written for one sequence must not be a slot that another
 * sequence of the batch reads as part of its cached prefix.  q, k_new, v_new
 * and the cached prefix must hold finite values.  Metadata is read on the
 * device only (check it with attn_validate_chunk_metadata, chunk_len = Tq).
 */
int attn_prefill_paged_append(const void* q, const void* k_new, const void* v_new,
                              void* k_pages, void* v_pages,
                              const int32_t* block_table, const int32_t* seq_lens,
                              void* out, float* lse,
                              int B, int Hq, int Hkv, int Tq, int d, int page_size, int num_pages,
                              int max_pages_per_seq, float scale, int dtype,
                              hipStream_t stream);

/*
 * Split plan of attn_decode_paged: a sequence's page list may be cut only at
 * multiples of pages_per_split = ceil(max_pages_per_seq / S), so it is cut
 * into at most S pieces; this returns S.  num_splits > 0 asks for that many
 * (clamped to max_pages_per_seq); num_splits == 0 lets the library choose
 * from the shape alone (no device query, no device read).  Returns S >= 1,
 * or a negative attn_status_t for invalid sizes.
 */
int attn_decode_num_splits(int B, int Hq, int Hkv, int d, int page_size,
                           int max_pages_per_seq, int num_splits);

/*
 * Bytes of device workspace attn_decode_paged needs for this shape: with
 * G = Hq / Hkv and P = B * Hkv + 4096 piece slots, fp32 partial outputs
 * [P, G, d], fp32 partial log-sum-exps [P, G] and four int32 per
 * (sequence, kv head), each region 256-byte aligned.  It grows with B, Hq
 * and d only: the sequence lengths, max_pages_per_seq and the split request
 * do not change it (the arguments are validated all the same).  Returns 0
 * for invalid sizes.
 */
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int page_size,
                                   int max_pages_per_seq, int num_splits);

/*
 * Single-token decode over a paged KV cache (split-KV + LSE combine).
 *
 *   q, out         : device, [B, Hq, d] in `dtype`
 *   k_pages,v_pages: device, [num_pages, Hkv, page_size, d] in `dtype`; the
 *                    (page, kv head) slice is contiguous (page_size*d values)
 *   block_table    : device int32 [B, max_pages_per_seq]; token j of sequence
 *                    b is slot j % page_size of page block_table[b][j / page_size].
 *                    Entries past ceil(seq_lens[b] / page_size) are never read.
 *   seq_lens       : device int32 [B]; cached tokens per sequence, each in
 *                    [0, max_pages_per_seq * page_size].  0 gives out = 0 and
 *                    lse = -inf for that sequence.
 *   lse            : device float32 [B, Hq], or NULL to skip it
 *   num_pages      : pool size; every block_table entry that is read must be
 *                    in [0, num_pages)
 *   num_splits     : as for attn_decode_num_splits (0 = automatic)
 *   workspace      : device, at least attn_decode_workspace_bytes(...) bytes;
 *                    owned by the caller, contents on entry are ignored
 *   dtype          : ATTN_BF16; d = 128 or 64; page_size = 16; Hq / Hkv <= 16;
 *                    B * Hkv * max_pages_per_seq < 2^31
 * Slots at or past seq_lens[b] may hold anything (NaN included): they are
 * never used.  The block table and seq_lens are read on the device only;
 * values outside the ranges above are undefined behaviour (check them with
 * attn_validate_paged_metadata).  Calls that share a workspace must not
 * overlap in time.
 */
int attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                      const int32_t* block_table, const int32_t* seq_lens,
                      void* out, float* lse,
                      int B, int Hq, int Hkv, int d, int page_size, int num_pages,
                      int max_pages_per_seq, float scale, int dtype,
                      int num_splits, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * Decode with the KV append fused: the work of attn_kv_append with Tn = 1
 * (k_new, v_new written at position seq_lens[b] - 1) followed by
 * attn_decode_paged, in the same two launches as the decode alone; out, lse
 * and the pools come out bit for bit as from those two calls (same
 * num_splits).  The split kernel reads the newest token from k_new / v_new,
 * not from its slot; the combine kernel, which runs after it, writes the
 * slot.
 *
 *   k_new, v_new   : device, [B, Hkv, d] (the layout of [B, Hkv, 1, d]): the
 *                    newest token's key and value per sequence and kv head
 *   k_pages,v_pages: as for attn_decode_paged; written only at the slot of
 *                    position seq_lens[b] - 1 of each sequence
 *   seq_lens       : lengths after the append; a sequence with 0 appends
 *                    nothing and decodes to out = 0, lse = -inf
 *   other arguments: as for attn_decode_paged (dtype ATTN_BF16 only)
 * Two sequences' newest tokens must not name the same (page, slot), and no
 * sequence may read another's newest-token slot as part of its cache.
 * Calls that share a workspace must not overlap in time.
 */
int attn_decode_paged_append(const void* q, const void* k_new, const void* v_new,
                             void* k_pages, void* v_pages,
                             const int32_t* block_table, const int32_t* seq_lens,
                             void* out, float* lse,
                             int B, int Hq, int Hkv, int d, int page_size, int num_pages,
                             int max_pages_per_seq, float scale, int dtype,
                             int num_splits, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * attn_decode_paged without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Arguments, layouts and results are
 * those of attn_decode_paged; the workspace is a static array of 64 MiB in
 * the library's device code, one per GPU, held from the library's load until
 * the process ends.  The call allocates and frees nothing.
 *
 * Limit: shapes whose attn_decode_workspace_bytes() exceeds 64 MiB (67108864
 * bytes) are rejected with ATTN_ERR_WORKSPACE before any HIP call: about
 * B * Hq * (d + 1) * 4 bytes plus 8.5 MB, so at Hq = 32, Hkv = 8, d = 128 up
 * to B = 3524 sequences.  No part of the scratch needs to start at zero
 * (every value a call reads, the call wrote first).
 * Every call on a GPU uses that GPU's one array: calls that overlap in time
 * on one GPU (on different streams, or from different threads) race and may
 * return wrong results; serialise them.
 */
int attn_decode_paged_noalloc(const void* q, const void* k_pages, const void* v_pages,
                              const int32_t* block_table, const int32_t* seq_lens,
                              void* out, float* lse,
                              int B, int Hq, int Hkv, int d, int page_size, int num_pages,
                              int max_pages_per_seq, float scale, int dtype,
                              int num_splits, hipStream_t stream);

/*
 * Single-token decode over a paged KV cache stored in FP8 E4M3.
 *
 *   k_pages,v_pages: device, [num_pages, Hkv, page_size, d] bytes, each an
 *                    FP8 E4M3 code (OCP 8-bit float: sign, 4-bit exponent with
 *                    bias 7, 3-bit mantissa, subnormals, no infinity, 0x7F and
 *                    0xFF NaN); the key at a slot is code value * k_scale, the
 *                    value code value * v_scale
 *   k_scale,v_scale: finite per-tensor scales
 * Every other argument, the workspace and the result are as for
 * attn_decode_paged (q, out, lse bf16 / fp32 as there; page_size = 16,
 * d = 128 or 64, Hq / Hkv <= 16).  Codes at slots past seq_lens[b] may hold
 * anything (NaN codes included); the cached codes of valid slots must not
 * be NaN.
 */
int attn_decode_paged_fp8(const void* q, const void* k_pages, const void* v_pages,
                          float k_scale, float v_scale,
                          const int32_t* block_table, const int32_t* seq_lens,
                          void* out, float* lse,
                          int B, int Hq, int Hkv, int d, int page_size, int num_pages,
                          int max_pages_per_seq, float scale, int num_splits,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Host-side check of paged metadata (host copies of block_table and
 * seq_lens): every seq_len in [0, max_pages_per_seq * page_size] and every
 * block-table entry that a sequence reads in [0, num_pages).  Returns ATTN_OK
 * or ATTN_ERR_INVALID_ARG.  Touches no device.
 */
int attn_validate_paged_metadata(const int32_t* block_table_host, const int32_t* seq_lens_host,
                                 int B, int max_pages_per_seq, int page_size, int num_pages);

/*
 * attn_validate_paged_metadata plus the chunked-prefill condition
 * seq_lens[b] >= chunk_len for every sequence.  Host only; touches no device.
 */
int attn_validate_chunk_metadata(const int32_t* block_table_host, const int32_t* seq_lens_host,
                                 int B, int max_pages_per_seq, int page_size, int num_pages,
                                 int chunk_len);

/* Static description of a status code (never NULL). */
const char* attn_status_string(int status);

/* Text describing the most recent failed call on this thread ("" if none). */
const char* attn_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
