/*
 * attn.h — C ABI of the MI355X (gfx950) masked / LSE / decode attention library.
 *
 * Exact scaled-dot-product attention that never materialises the
 * heads x Tq x Tk score matrix.  Every call only enqueues HIP kernels on the
 * caller's stream and returns; there is no host synchronisation, no device
 * allocation and no pointer retained after return.
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller, dense and
 *     row-major in the layouts stated below, 16-byte aligned.
 *   - `dtype` is ATTN_F32 (float) or ATTN_BF16 (bfloat16); all tensor
 *     operands of one call share it, except LSE arrays, which are always
 *     float32, the mask (uint8) and cache lengths (int32).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every kernel of a call goes to that stream, so calls may be captured into
 *     a HIP graph.  The first call of an entry point on a device does one-time
 *     set-up (kernel attributes, an occupancy query, the static scratch's
 *     address); make that first call outside a capture.
 *   - Head dimension D must be 64 or 128.
 *   - No output may share a byte with an input or with another output (byte
 *     ranges from the stated shapes; in-place use is refused, ATTN_ERR_ALIAS).
 *   - Return value: an attn_status.  Argument checks happen on the host
 *     before anything is enqueued; a failed check enqueues nothing.  A
 *     launch failure reported by hipGetLastError maps to ATTN_ERR_LAUNCH.
 *   - Arithmetic: bf16 inputs feed bf16 matrix-core products with float32
 *     accumulation; the softmax statistics, normalisation and LSE are float32;
 *     bf16 outputs are rounded to nearest even.  float32 inputs are computed
 *     in float32 throughout.
 */
#ifndef MASKED_ATTN_ATTN_H
#define MASKED_ATTN_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_F32 = 0,
    ATTN_BF16 = 1
} attn_dtype;

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,         /* a required pointer is NULL */
    ATTN_ERR_SHAPE = 2,        /* a size is out of range or inconsistent */
    ATTN_ERR_UNSUPPORTED = 3,  /* D not in {64,128}, unknown dtype, too many chunks */
    ATTN_ERR_WORKSPACE = 4,    /* decode workspace missing or too small */
    ATTN_ERR_LAUNCH = 5,       /* hipGetLastError reported a failure after enqueueing */
    ATTN_ERR_VALUE = 6,        /* scale is not a finite positive number */
    ATTN_ERR_ALIGN = 7,        /* a tensor pointer is not 16-byte aligned */
    ATTN_ERR_ALIAS = 8,        /* an output's bytes overlap an input or another output */
    ATTN_ERR_SCRATCH = 9       /* attn_decode_noalloc: more scratch needed than its static buffer */
} attn_status;

/*
 * attn_fwd_masked — non-causal masked attention, O = softmax(scale·Q·Kᵀ + pad)·V.
 *
 * Defines the operation the MultiheadAttention inference fast path computes
 * with a key-padding mask (molayo1419.me, "MultiheadAttention의 고속 경로가
 * VRAM을 18GB나 소모했던 이야기", section "소스의 현실": scores [B, heads,
 * T, T], masked softmax, product with V), computed here tile by tile so
 * that only O(Tq + Tk) extra memory exists; padding acts as an additive -inf
 * on the scores of padded keys (same page, "CPU에서 양을 측정하기").
 *
 *   q    [B, H, Tq, D]   queries
 *   k, v [B, H, Tk, D]   keys and values
 *   key_padding_mask  [B, Tk] uint8; NONZERO = padded = ignored (the
 *        key_padding_mask polarity, the opposite of a boolean SDPA mask; same
 *        page, "출력은 달라졌는가").  NULL = no padding.  Values stored at
 *        padded keys are ignored but V there must be finite.
 *   o    [B, H, Tq, D]   output, same dtype as q
 *   scale  multiplier of Q·Kᵀ, finite and > 0 (usually 1/sqrt(D))
 * Sizes: B, H, Tq, Tk >= 1; bf16: Tk·D·2 below 2^31 (one head's K or V is
 * addressed through a 32-bit range), else ATTN_ERR_SHAPE.  A query whose keys
 * are all padded gets O = 0.  Queries are never masked: every query row is
 * computed.
 */
int attn_fwd_masked(const void* q, const void* k, const void* v,
                    const uint8_t* key_padding_mask, void* o,
                    int B, int H, int Tq, int Tk, int D,
                    float scale, int dtype, void* stream);

/*
 * attn_fwd_lse — attn_fwd_masked that also writes the per-row log-sum-exp.
 *
 * The LSE is what an online-softmax merge of results over separate KV
 * chunks needs (blog.secrett2633.cloud, sglang PR 49078 analysis, section
 * "1. aiter.py — LSE 반환과 ring 지원 선언").
 *   lse [B, H, Tq] float32: natural-log log-sum-exp over unpadded keys of the
 *       scaled scores, lse = log sum_j exp(scale·q·k_j); -inf for a row with
 *       no unpadded key.
 * All other arguments as attn_fwd_masked.
 */
int attn_fwd_lse(const void* q, const void* k, const void* v,
                 const uint8_t* key_padding_mask, void* o, float* lse,
                 int B, int H, int Tq, int Tk, int D,
                 float scale, int dtype, void* stream);

/*
 * attn_fwd_varlen — attention of packed variable-length sequences, with LSE.
 *
 * The packed call a ring-attention hop makes (sglang PR 49078 analysis,
 * section "1. aiter.py", forward_ring_kv_chunk): a [T, H, D] query attends
 * a KV chunk, sequences delimited by cumulative-length arrays, non-causal,
 * returning the LSE as [H, Tq].  Sequence b owns query rows
 * [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key rows [cu_seqlens_k[b],
 * cu_seqlens_k[b+1]); its queries attend exactly its keys (no mask: the
 * packing replaces padding).
 *   q, o  [total_q, H, D] bf16      k, v  [total_k, H, D] bf16
 *   cu_seqlens_q, cu_seqlens_k  [B+1] int32 device arrays, non-decreasing from
 *       0 to total; owned by the caller and only read (same page: the cached
 *       cu_seqlens tensors must not be mutated).  Entries are clamped to
 *       [0, total], so a malformed array gives wrong rows but no access out
 *       of range.
 *   lse   [H, total_q] float32 (natural log) or NULL; -inf for a query whose
 *       sequence has no keys (its O row is 0)
 *   max_seqlen_q  at least the longest query sequence (it sizes the grid;
 *       rows past it are not written); 0 <= max_seqlen_q <= total_q
 * bf16 only (ATTN_ERR_UNSUPPORTED otherwise); H·D <= 2^22, total_k·H·D < 2^30
 * and total_q·H·D < 2^31 (else ATTN_ERR_SHAPE); the other rules as
 * attn_fwd_masked.  total_q = 0 or max_seqlen_q = 0 is a no-op; with total_k = 0 (no keys:
 * every row gets O = 0, LSE = -inf) k and v may be NULL.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                    void* o, float* lse,
                    int B, int H, int total_q, int total_k, int max_seqlen_q, int D,
                    float scale, int dtype, void* stream);

/*
 * attn_prefill — grouped-query, optionally causal attention (the prompt pass).
 *
 * The prefill phase of a grouped-query-attention language model: the whole
 * prompt is encoded once and its K/V fill the cache (nanoVLM-KV page,
 * agentlenshq.com "nanoVLM에서 KV 캐시 구현", sections "1. 어텐션 블록
 * 업데이트" and "3. 생성 루프 분리"); query heads share KV heads (LLM
 * inference memory accounting 2/10, "11. 계산 예시: GQA Decoder").
 *   q, o  [B, H_q, Tq, D] bf16      k, v  [B, H_kv, Tk, D] bf16
 *   query head h reads KV head h / (H_q / H_kv); H_q must be a multiple of H_kv
 *   causal  nonzero: query i sees keys j <= i + (Tk - Tq) only, i.e. the Tq
 *       queries are the last Tq of the Tk positions (Tq = Tk: j <= i; Tq = 1:
 *       every key).  A query that sees no key gets O = 0, LSE = -inf.
 *   key_padding_mask  [B, Tk] uint8 or NULL, as attn_fwd_masked (combined
 *       with the causal limit)
 *   lse  [B, H_q, Tq] float32 or NULL
 * bf16 only when causal or H_kv != H_q (ATTN_ERR_UNSUPPORTED otherwise; with
 * neither it is attn_fwd_masked / attn_fwd_lse and takes float32 too).  Other
 * rules as attn_fwd_masked.
 */
int attn_prefill(const void* q, const void* k, const void* v,
                 const uint8_t* key_padding_mask, void* o, float* lse,
                 int B, int H_q, int H_kv, int Tq, int Tk, int D, int causal,
                 float scale, int dtype, void* stream);

/*
 * attn_prefill_varlen — attn_prefill on packed sequences.
 *
 * The varlen call with its causal flag (sglang PR 49078 analysis, section
 * "1. aiter.py": flash_attn_varlen_func takes cu_seqlens and causal; the
 * ring hop passes causal = false).  Layouts, cu_seqlens, LSE [H_q, total_q]
 * and max_seqlen_q as attn_fwd_varlen, with k, v [total_k, H_kv, D]; the
 * causal limit uses each sequence's own lengths.  bf16 only; H_q·D <= 2^22,
 * total_k·H_kv·D < 2^30, total_q·H_q·D < 2^31.
 */
int attn_prefill_varlen(const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        void* o, float* lse,
                        int B, int H_q, int H_kv, int total_q, int total_k, int max_seqlen_q,
                        int D, int causal, float scale, int dtype, void* stream);

/*
 * attn_merge_lse — combine n partial results over disjoint KV chunks.
 *
 * out = sum_i exp(lse_i - lse)·out_i with lse = log sum_i exp(lse_i), the
 * merge ring attention applies per hop (sglang PR 49078 analysis, section
 * "1. aiter.py"); rows with every lse_i = -inf give out = 0, lse = -inf.
 *   n_chunks  1..32
 *   outs  HOST array of n_chunks device pointers, each [B, H, T, D] (dtype)
 *   lses  HOST array of n_chunks device pointers, each [B, H, T] float32
 *   out   [B, H, T, D] (dtype); must not be any outs[i] (nor lse_out any lses[i])
 *   lse_out  [B, H, T] float32, or NULL to skip
 */
int attn_merge_lse(int n_chunks, const void* const* outs, const float* const* lses,
                   void* out, float* lse_out,
                   int B, int H, int T, int D, int dtype, void* stream);

/*
 * kv_append — append one token per sequence to preallocated K/V caches.
 *
 * After the prompt is cached, each decode step computes K and V only for
 * the newest token and adds them to the cache (agentlenshq.com, "nanoVLM에서
 * KV 캐시 구현", sections "KV 캐싱이 추론을 최적화하는 방법" and
 * "1. 어텐션 블록 업데이트"; cache tensors are (batch, heads, seq_len_cached,
 * head_dim)).  Here the cache has fixed capacity T_max and appending writes
 * slot cache_seqlens[b] and then increments it.
 *   k_cache, v_cache  [B, H_kv, T_max, D] (dtype), modified in place
 *   cache_seqlens     [B] int32 device array, read then incremented in place
 *   k_new, v_new      [B, H_kv, 1, D] (dtype)
 * A sequence whose length is < 0 or >= T_max is left untouched (no write,
 * no increment); keeping len < T_max is the caller's responsibility.
 */
int kv_append(void* k_cache, void* v_cache, int32_t* cache_seqlens,
              const void* k_new, const void* v_new,
              int B, int H_kv, int T_max, int D, int dtype, void* stream);

/*
 * attn_decode — one query token per sequence against the KV cache (GQA).
 *
 * The current token's query attends over every cached position (nanoVLM
 * KV-cache page, "KV 캐싱이 추론을 최적화하는 방법"); the bytes that must be
 * read are 2·H_kv·D·elem_bytes per cached token (blog.ruahverce.com, LLM
 * inference memory accounting 2/10, sections "10. KV Cache Byte 공식" and
 * "13. KV는 Token마다 자란다"), and query heads that share a KV head share
 * its reads (same page, "11. 계산 예시: GQA Decoder").
 *   q   [B, H_q, 1, D]; query head h uses KV head h / (H_q / H_kv)
 *   k_cache, v_cache  [B, H_kv, T_max, D]
 *   cache_seqlens [B] int32 device: positions 0..len-1 are attended
 *       (len = 0 gives O = 0, LSE = -inf; a length outside [0, T_max] is
 *       clamped to that range)
 *   o   [B, H_q, 1, D] (dtype);  lse [B, H_q] float32 or NULL
 *   workspace  device scratch of at least attn_decode_workspace_bytes(...)
 *       bytes, owned by the caller, 16-byte aligned; contents on entry are
 *       ignored and are garbage on return.  Calls that share a workspace
 *       must be ordered on one stream.
 * H_q must be a multiple of H_kv.  bf16: T_max·D·2 must stay below 2^31 (one
 * (sequence, KV head) is addressed through a 32-bit range), else
 * ATTN_ERR_SHAPE.
 */
int attn_decode(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* cache_seqlens, void* o, float* lse,
                int B, int H_q, int H_kv, int T_max, int D,
                float scale, int dtype,
                void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace attn_decode needs for these sizes (0 on invalid sizes).
 * attn_decode_paged needs the same with T_max = max_pages_per_seq · page_size. */
size_t attn_decode_workspace_bytes(int B, int H_q, int H_kv, int T_max, int D);

/*
 * attn_decode_noalloc — attn_decode for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, checks and results as attn_decode, without the workspace: the partial
 * results live in a static device buffer of ATTN_DECODE_NOALLOC_SCRATCH_BYTES inside the
 * library (one per GPU the library runs on, held until the process ends).  The call
 * allocates nothing, takes the buffer's device address once per device on its first call
 * there (hipGetSymbolAddress), and then only enqueues the attn_decode kernels.
 *   Limit: attn_decode_workspace_bytes(B, H_q, H_kv, T_max, D) must not exceed
 *       ATTN_DECODE_NOALLOC_SCRATCH_BYTES, else ATTN_ERR_SCRATCH (nothing enqueued).  At
 *       D = 128 that is B·H_q·ceil(T_max / 1024) <= 32,263 (e.g. 32 sequences x 32 query
 *       heads up to T_max = 31,744).
 *   Every call on one GPU shares that GPU's buffer, which keeps the last call's contents
 *   (nothing in it needs clearing: every slot a call reads, the same call writes first).
 *   Calls that overlap in time on one GPU (different streams, no ordering) race on it;
 *   order them on one stream.
 */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* cache_seqlens, void* o, float* lse,
                        int B, int H_q, int H_kv, int T_max, int D,
                        float scale, int dtype, void* stream);

/*
 * Paged KV cache.  A sequence's logical KV blocks live in non-contiguous
 * physical blocks of a shared pool, found through its row of a block table
 * (blog.ruahverce.com, LLM inference memory accounting 2/10, section
 * "15. Paged KV Cache가 해결하는 것": logical block i of a request maps to
 * physical block block_table[i]; the attention kernel must read that
 * layout).  Conventions of the two paged calls:
 *   k_pages, v_pages  [num_pages, H_kv, page_size, D] (dtype): a physical page
 *       holds page_size consecutive tokens of every KV head, each head's
 *       page_size rows contiguous
 *   block_table  [B, max_pages_per_seq] int32 device array, owned by the
 *       caller and only read: token t of sequence b is row t % page_size of
 *       page block_table[b][t / page_size].  Only the entries covering
 *       positions 0..len_b (decode: 0..len_b - 1) are read; an entry outside
 *       [0, num_pages) is clamped into it (wrong values, no access outside
 *       the pool).  Pages may be shared between sequences.
 *   page_size  a power of two, 16 <= page_size <= 2^20
 *   capacity   T_max = max_pages_per_seq · page_size <= 2^30 tokens; B ·
 *       max_pages_per_seq <= 2^29
 * Lengths, q, o, lse, scale, workspace and errors as the contiguous calls.
 */

/* kv_append_paged — kv_append into a paged cache: the new token of sequence
 * b is written at row len_b % page_size of page block_table[b][len_b /
 * page_size], then len_b is incremented; a length outside [0, T_max) leaves
 * the sequence untouched.  k_new, v_new [B, H_kv, 1, D] (dtype). */
int kv_append_paged(void* k_pages, void* v_pages, const int32_t* block_table,
                    int32_t* cache_seqlens, const void* k_new, const void* v_new,
                    int B, int H_kv, int num_pages, int page_size, int max_pages_per_seq,
                    int D, int dtype, void* stream);

/* attn_decode_paged — attn_decode over a paged cache (bf16 only, else
 * ATTN_ERR_UNSUPPORTED): the same result as attn_decode over the contiguous
 * cache that the block table describes.  workspace as attn_decode with
 * T_max = max_pages_per_seq · page_size. */
int attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                      const int32_t* block_table, const int32_t* cache_seqlens,
                      void* o, float* lse,
                      int B, int H_q, int H_kv, int num_pages, int page_size,
                      int max_pages_per_seq, int D, float scale, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * FP8 (E4M3) KV cache.  KV-cache quantisation stores each cached element in
 * fewer bytes plus scale metadata and dequantises inside the attention kernel
 * (blog.ruahverce.com, LLM inference memory accounting 2/10, section
 * "18. KV Quantization은 Byte와 Kernel을 함께 바꾼다").  Layout and conventions of the two FP8 calls:
 *   k_cache, v_cache  [B, H_kv, T_max, D] uint8: OCP E4M3 codes (1 sign, 4
 *       exponent bits with bias 7, 3 mantissa bits, subnormals, largest
 *       magnitude 448, S.1111.111 = NaN; no infinities)
 *   k_scale, v_scale  [B, H_kv] float32 device arrays, owned by the caller and
 *       only read: the cached element is code value x scale of its (sequence,
 *       KV head); scales must be finite and > 0
 *   q, o bf16 as in attn_decode; lengths, lse, workspace (attn_decode_workspace_bytes
 *   with the same sizes) and errors as attn_decode.
 */

/* kv_append_fp8 — quantise one token per sequence into slot cache_seqlens[b]:
 * code = E4M3(clamp(x / scale, -448, 448)) with x the new element as float32,
 * an IEEE float32 division and rounding to nearest, ties to even; then
 * cache_seqlens[b] += 1 (a length outside [0, T_max) leaves the sequence
 * untouched).  k_new, v_new [B, H_kv, 1, D] of new_dtype (ATTN_BF16 or ATTN_F32). */
int kv_append_fp8(void* k_cache, void* v_cache, const float* k_scale, const float* v_scale,
                  int32_t* cache_seqlens, const void* k_new, const void* v_new,
                  int B, int H_kv, int T_max, int D, int new_dtype, void* stream);

/* attn_decode_fp8kv — attn_decode against the FP8 cache: the same result as
 * attn_decode over the dequantised cache (codes are converted exactly to bf16,
 * the K scale multiplies the scores and the V scale the output).  T_max·D must
 * stay below 2^31. */
int attn_decode_fp8kv(const void* q, const void* k_cache, const void* v_cache,
                      const float* k_scale, const float* v_scale,
                      const int32_t* cache_seqlens, void* o, float* lse,
                      int B, int H_q, int H_kv, int T_max, int D, float scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * INT8 KV cache: the two FP8 calls above with symmetric INT8 codes, another of
 * the cache formats LLM inference memory accounting 2/10 lists (section
 * "18. KV Quantization은 Byte와 Kernel을 함께 바꾼다").
 *   k_cache, v_cache  [B, H_kv, T_max, D] int8: code q stands for q x scale
 *   k_scale, v_scale  as for the FP8 cache
 * kv_append_int8 writes code = clamp(rint(x / scale), -127, 127): an IEEE
 * float32 division, the nearest integer with ties to even, the symmetric range
 * (-128 is never written; a -128 in the cache decodes as -128).
 * attn_decode_int8kv returns attn_decode over the dequantised cache (codes are
 * converted exactly to bf16).  Lengths, lse, workspace, sizes and errors as
 * the FP8 calls.
 */
int kv_append_int8(void* k_cache, void* v_cache, const float* k_scale, const float* v_scale,
                   int32_t* cache_seqlens, const void* k_new, const void* v_new,
                   int B, int H_kv, int T_max, int D, int new_dtype, void* stream);

int attn_decode_int8kv(const void* q, const void* k_cache, const void* v_cache,
                       const float* k_scale, const float* v_scale,
                       const int32_t* cache_seqlens, void* o, float* lse,
                       int B, int H_q, int H_kv, int T_max, int D, float scale,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Paged 8-bit caches: the FP8 and INT8 calls above over page pools, the paged
 * layout of attn_decode_paged (LLM inference memory accounting 2/10, sections
 * "15. Paged KV Cache가 해결하는 것" and
 * "18. KV Quantization은 Byte와 Kernel을 함께 바꾼다").
 *   k_pages, v_pages  [num_pages, H_kv, page_size, D] codes (uint8 E4M3 or int8)
 *   block_table, page_size, max_pages_per_seq  as attn_decode_paged (T_max =
 *       max_pages_per_seq · page_size; the workspace is sized with that T_max)
 *   k_scale, v_scale  [B, H_kv] float32, per (sequence, KV head), as the contiguous calls
 * Quantisation, results and errors as the contiguous 8-bit calls; paging rules
 * (page sizes, clamped table entries) as the bf16 paged calls.
 */
int kv_append_fp8_paged(void* k_pages, void* v_pages, const float* k_scale, const float* v_scale,
                        const int32_t* block_table, int32_t* cache_seqlens,
                        const void* k_new, const void* v_new, int B, int H_kv, int num_pages,
                        int page_size, int max_pages_per_seq, int D, int new_dtype, void* stream);

int kv_append_int8_paged(void* k_pages, void* v_pages, const float* k_scale, const float* v_scale,
                         const int32_t* block_table, int32_t* cache_seqlens,
                         const void* k_new, const void* v_new, int B, int H_kv, int num_pages,
                         int page_size, int max_pages_per_seq, int D, int new_dtype, void* stream);

int attn_decode_fp8kv_paged(const void* q, const void* k_pages, const void* v_pages,
                            const float* k_scale, const float* v_scale, const int32_t* block_table,
                            const int32_t* cache_seqlens, void* o, float* lse, int B, int H_q,
                            int H_kv, int num_pages, int page_size, int max_pages_per_seq, int D,
                            float scale, void* workspace, size_t workspace_bytes, void* stream);

int attn_decode_int8kv_paged(const void* q, const void* k_pages, const void* v_pages,
                             const float* k_scale, const float* v_scale, const int32_t* block_table,
                             const int32_t* cache_seqlens, void* o, float* lse, int B, int H_q,
                             int H_kv, int num_pages, int page_size, int max_pages_per_seq, int D,
                             float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_prefill_fp8 — attn_prefill on E4M3 inputs, with the LSE.
 *
 * The aiter ring-attention analysis (sglang PR 49078 analysis, section
 * "1. aiter.py") notes that the FP8 prefill kernel there has no LSE output, so
 * a ring hop that needs the LSE stays in BF16; this call returns it.  The
 * result is attn_prefill (GQA, optional key padding, optional causal limit)
 * on the dequantised inputs:
 *   q  [B, H_q, Tq, D] uint8      k, v  [B, H_kv, Tk, D] uint8: E4M3 codes as
 *       in the FP8 cache above (NaN codes are not valid input)
 *   q_scale [B, H_q], k_scale and v_scale [B, H_kv] float32 device arrays,
 *       owned by the caller and only read: an element stands for code value x
 *       the scale of its (sequence, head); scales must be finite and > 0
 *   o  [B, H_q, Tq, D] bf16        lse  [B, H_q, Tq] float32 or NULL
 *   key_padding_mask, causal, scale  as attn_prefill
 * Q·Kᵀ runs on the E4M3 matrix cores (exact products, float32 sums); the
 * softmax weights and P·V are bf16 as in attn_prefill.  Tk·D must stay below
 * 2^31; other rules and errors as attn_prefill.
 */
int attn_prefill_fp8(const void* q, const void* k, const void* v,
                     const float* q_scale, const float* k_scale, const float* v_scale,
                     const uint8_t* key_padding_mask, void* o, float* lse,
                     int B, int H_q, int H_kv, int Tq, int Tk, int D, int causal,
                     float scale, void* stream);

/*
 * attn_prefill_varlen_fp8 — attn_prefill_varlen on E4M3 inputs, with the LSE: the packed call a
 * ring-attention hop makes (sglang PR 49078 analysis, section "1. aiter.py"), in the FP8 form
 * that analysis finds without an LSE output.  Layouts as attn_prefill_varlen with uint8 codes
 * for q [total_q, H_q, D] and k, v [total_k, H_kv, D]; q_scale [B, H_q], k_scale and v_scale
 * [B, H_kv] float32, one per (sequence, head), as attn_prefill_fp8; o [total_q, H_q, D] bf16,
 * lse [H_q, total_q] float32 or NULL.  Size limits and errors as attn_prefill_varlen;
 * total_q = 0 or max_seqlen_q = 0 is a no-op.
 */
int attn_prefill_varlen_fp8(const void* q, const void* k, const void* v,
                            const float* q_scale, const float* k_scale, const float* v_scale,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            void* o, float* lse, int B, int H_q, int H_kv,
                            int total_q, int total_k, int max_seqlen_q, int D, int causal,
                            float scale, void* stream);

/* Static, human-readable name of a status code. */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MASKED_ATTN_ATTN_H */
