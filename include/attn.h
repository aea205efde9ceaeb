/*
 * attn.h — flash-attention forward for AMD Instinct MI355X (gfx950), C ABI.
 *
 * Three entry points compute softmax attention
 *
 *     O = softmax(scale * Q K^T  restricted to the visible keys) V
 *
 * with the online-softmax recurrence (running row max m, running sum l,
 * rescale alpha = exp(m_old - m_new) of O and l, final O * (1/l)):
 *   - attn_prefill_fwd     long Q against K/V of the same sequence (compute bound),
 *                          with _ex (lse output, sinks), _varlen (packed sequences)
 *                          and _fp8kv (K and V stored as FP8 E4M3);
 *   - attn_decode_fwd      a few query tokens against a long, optionally paged,
 *                          KV cache, split along the cache into partial results
 *                          (_fp8kv: an FP8 E4M3 cache);
 *   - attn_decode_combine  the log-sum-exp merge of those partials (_ex: lse, sinks).
 * Helpers: attn_decode_workspace_size, attn_decode_validate_pages (a device-side
 * check of a page table) and attn_status_string.
 *
 * The recurrence and its final normalisation are the ones described on the
 * "Flash-Attention: Context (CTE)" page (section "The online-softmax
 * recurrence") and on the minfer "03 · 8n — FA-style tiled prefill attention"
 * page (section 2.1 "Online softmax").
 *
 * Conventions shared by all entry points
 * --------------------------------------
 * Tensors are row-major with element strides; the head_dim stride is 1.
 *   q, o     : [batch, seqlen_q, n_q_heads, head_dim]
 *   k, v     : [batch, seqlen_kv, n_kv_heads, head_dim]
 * GQA: q-head h reads kv-head h / (n_q_heads / n_kv_heads); n_q_heads must
 * be a multiple of n_kv_heads (CTE page, section "GQA and multi-head").
 * Query row i sits at position i + (seqlen_kv - seqlen_q) (bottom-right
 * alignment, so a decode query sits at the end of its cache). Key j is
 * visible to row i iff
 *     (!causal || j <= pos(i))  &&  (window <= 0 || j >= pos(i) - window + 1)
 * (causal predicate: CTE page, "the diagonal affine_select mask"; window
 * predicate: optimum-neuron attention guide, section "Sliding window";
 * window <= 0 means no window, as that guide's default). A row that sees no
 * key outputs zeros. `scale` multiplies the scores (CTE page, section
 * "Scale"); the library never divides by sqrt(head_dim) itself.
 *
 * Finite inputs: Q, and K and V at every key some query row of the call
 * sees, must be finite. Masked keys add exactly nothing for finite data,
 * bit for bit, also inside the tiles that straddle the diagonal or the
 * window edge; but a masked key's value row still enters the P*V product of
 * its tile with probability 0, so a NaN or Inf value there can turn rows of
 * the same query tile NaN that the plain definition leaves finite. Keys at
 * or past seqlen_kv (cache_len), keys before the window of the call's
 * earliest query row and cache pages the table does not reference are never
 * read, so any bits there are harmless.
 *
 * Supported: head_dim in {64, 128, 256}; dtype f32, f16 or bf16 for Q, K, V
 * and O alike (f32 accumulation throughout; probabilities are rounded to
 * the input dtype before the P*V product for f16/bf16).
 *
 * Memory and streams: every pointer argument named a tensor is a device
 * pointer (hipMalloc / torch CUDA memory); the caller owns all of them and
 * the library allocates nothing and keeps no state between calls. Work is
 * enqueued on `hip_stream` (a hipStream_t; NULL = the default stream) and
 * the functions return without synchronising. Base pointers must be 16-byte
 * aligned and every stride times the element size must be a multiple of 16
 * bytes.
 *
 * Errors: all host-checkable preconditions are validated before any HIP
 * call; a violation returns ATTN_ERR_INVALID or ATTN_ERR_UNSUPPORTED and
 * enqueues nothing. A failed launch returns ATTN_ERR_LAUNCH after the HIP
 * error state has been read and cleared, so no sticky error is left behind
 * (the minfer page's pitfall about clearing a failed launch's error).
 * Zero-sized problems return ATTN_OK and enqueue nothing. Device-side data
 * (block tables, cache lengths) is not validated: out-of-range page indices
 * are undefined behaviour, as the decode page's gather treats them as a
 * fault ("Flash-Attention: Decode (TKG)", section "Paged / block cache").
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_F32 = 0, ATTN_F16 = 1, ATTN_BF16 = 2 } attn_dtype;

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID = 1,     /* malformed arguments (sizes, strides, alignment, NULL) */
    ATTN_ERR_UNSUPPORTED = 2, /* well-formed but not implemented (head_dim, dtype, mask combination) */
    ATTN_ERR_LAUNCH = 3       /* the HIP runtime rejected a launch */
} attn_status;

/* Element strides of a 4-D [batch, seq, head, head_dim] tensor. */
typedef struct {
    int64_t batch, seq, head;
} attn_strides;

/*
 * Prefill / context attention.
 *   q [batch, seqlen_q, n_q_heads, head_dim], k and v [batch, seqlen_kv,
 *   n_kv_heads, head_dim], o [batch, seqlen_q, n_q_heads, head_dim], all of
 *   type `dtype`, device memory, addressed through the given strides.
 *   causal != 0 enables the causal mask; window > 0 (requires causal) adds
 *   the sliding window. window > 0 without causal -> ATTN_ERR_UNSUPPORTED.
 * Whole tiles of keys that no query of a tile can see are skipped; only
 * tiles that straddle the diagonal or the window edge are masked element by
 * element (CTE page, "Algorithm — compute-skip" and the affine_select masks).
 */
int attn_prefill_fwd(const void* q, attn_strides q_st, const void* k, attn_strides k_st,
                     const void* v, attn_strides v_st, void* o, attn_strides o_st,
                     attn_dtype dtype, int batch, int n_q_heads, int n_kv_heads,
                     int seqlen_q, int seqlen_kv, int head_dim,
                     float scale, int causal, int window, void* hip_stream);

/*
 * attn_prefill_fwd with two optional extras (NULL = not used):
 *   lse    device float [batch, seqlen_q, n_q_heads] (contiguous): for every
 *          row, the natural-log log-sum-exp of its scaled visible scores
 *          (and of the sink), m + log(l) — the softmax statistics the CTE
 *          page writes out for a backward pass ("cache_softmax": the row max
 *          and the reciprocal of the sum) and what a sequence-parallel merge
 *          needs. -inf for a row that sees no key and has no sink.
 *   sinks  device float [n_q_heads]: an attention sink per q-head — one more
 *          logit of every row of that head, in the units of the scaled
 *          scores, that joins the row max and the softmax sum but has no
 *          value row (CTE page: the sink logit appended to the section max
 *          and its exponential to the sums; decode page: one sink per q-head,
 *          broadcast over the batch). O becomes sum_j p_j v_j / (sum_j p_j +
 *          exp(sink - m)). A sink of -inf is no sink; NaN or +inf sinks give
 *          NaN rows. A row that sees no key outputs zeros and lse = sink.
 * Both pointers must be 4-byte aligned.
 */
int attn_prefill_fwd_ex(const void* q, attn_strides q_st, const void* k, attn_strides k_st,
                        const void* v, attn_strides v_st, void* o, attn_strides o_st,
                        attn_dtype dtype, int batch, int n_q_heads, int n_kv_heads,
                        int seqlen_q, int seqlen_kv, int head_dim,
                        float scale, int causal, int window,
                        float* lse, const float* sinks, void* hip_stream);

/*
 * attn_prefill_fwd_ex with K and V stored in FP8 E4M3 (the OCP "e4m3fn"
 * encoding, as for attn_decode_fwd_fp8kv): the decode page's FP8-e4m3 cache
 * ("Flash-Attention: Decode (TKG)", section "KV-cache layouts and access")
 * read by the prefill, e.g. a chunk of new tokens attending to a cached FP8
 * prefix. k and v hold one byte per element in the [batch, seqlen_kv,
 * n_kv_heads, head_dim] layout with strides in elements (bytes); each row
 * must start 16-byte aligned. A stored code x stands for k_scale * value(x)
 * (K) or v_scale * value(x) (V). q and o are `dtype` (f16 or bf16; f32 is
 * ATTN_ERR_UNSUPPORTED), and shapes, masks, lse and sinks are as for
 * attn_prefill_fwd_ex. The codes are widened exactly to the 16-bit type of q
 * before the products, so the only rounding beyond attn_prefill_fwd_ex is the
 * cache's own. k_scale, v_scale and scale * k_scale must be finite (else
 * ATTN_ERR_INVALID); NaN codes give NaN rows.
 */
int attn_prefill_fwd_fp8kv(const void* q, attn_strides q_st, const uint8_t* k, attn_strides k_st,
                           const uint8_t* v, attn_strides v_st, void* o, attn_strides o_st,
                           attn_dtype dtype, int batch, int n_q_heads, int n_kv_heads,
                           int seqlen_q, int seqlen_kv, int head_dim,
                           float scale, float k_scale, float v_scale, int causal, int window,
                           float* lse, const float* sinks, void* hip_stream);

/*
 * Prefill over packed sequences of different lengths (sequence packing):
 * the bounds of every sequence are data, not shapes (the CTE page's dynamic
 * range_select family, section "Algorithm — the dynamic range_select
 * family": sequence-packing bounds and a dynamic prefix length; the minfer
 * page's kernel, section 3.1, reads the key bound from its positions input).
 *   q, o   [total_q, n_q_heads, head_dim] and k, v [total_kv, n_kv_heads,
 *          head_dim], device, `dtype`, addressed with the seq and head
 *          strides of q_st, k_st, v_st, o_st (their batch strides are ignored).
 *   cu_seqlens_q, cu_seqlens_kv  device int32 [batch + 1], nondecreasing:
 *          sequence b owns q/o rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) and
 *          k/v rows [cu_seqlens_kv[b], cu_seqlens_kv[b+1]).
 *   max_seqlen_q, max_seqlen_kv  at least every sequence's q and k/v length
 *          (the launch covers max_seqlen_q rows per sequence; rows of a longer
 *          sequence beyond it are not computed).
 * Within each sequence the usual rules hold: its query row i sits at position
 * i + (len_kv - len_q) (so len_q < len_kv is a chunk of new tokens after a
 * cached prefix), causal and window apply to those positions, GQA and the
 * optional lse ([total_q, n_q_heads], natural log) and sinks are as for
 * attn_prefill_fwd_ex. A sequence with no query rows writes nothing; one
 * with no keys outputs zeros.
 *   positions  NULL, or device int32 [total_q] (4-byte aligned): the position
 *          of every packed query row within its sequence's keys, replacing
 *          i + (len_kv - len_q) — the positions input of the minfer page's
 *          kernel (section 3.1: the key bound is the position of the tile's
 *          last row plus one, and key j is visible to a row at position P iff
 *          j <= P). Causal and window apply to these positions; they must be
 *          nondecreasing within each sequence (the tile bounds are taken from
 *          a tile's first and last rows). A position at or past len_kv sees
 *          all keys; a negative one sees none.
 * The offsets and positions are not validated on the host: offsets outside
 * the tensors are undefined behaviour.
 */
int attn_prefill_varlen_fwd(const void* q, attn_strides q_st, const void* k, attn_strides k_st,
                            const void* v, attn_strides v_st, void* o, attn_strides o_st,
                            attn_dtype dtype, int batch, int n_q_heads, int n_kv_heads,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                            int max_seqlen_q, int max_seqlen_kv, int head_dim,
                            float scale, int causal, int window,
                            float* lse, const float* sinks, const int32_t* positions,
                            void* hip_stream);

/*
 * Decode attention against a KV cache, split along the cache (split-KV).
 *   q       [batch, s_active, n_q_heads, head_dim] device, `dtype`.
 *   Paged cache (block_table != NULL): k_cache, v_cache are
 *           [num_pages, page_size, n_kv_heads, head_dim] with kv_st =
 *           (page, slot, head) strides; block_table is device uint32
 *           [batch, max_pages_per_seq]: logical token t of sequence b lives
 *           in physical page block_table[b*max_pages_per_seq + t/page_size],
 *           slot t%page_size (the decode page's `active_blocks_table`,
 *           section "Paged / block cache").
 *   Flat cache (block_table == NULL): k_cache, v_cache are
 *           [batch, >= cache_len[b], n_kv_heads, head_dim] with kv_st =
 *           (batch, seq, head); max_pages_per_seq and page_size are ignored.
 *   cache_len  device int32 [batch]: valid cache tokens per sequence,
 *           including the s_active current tokens, which the caller has
 *           already written. Keys with index >= cache_len[b] are never used
 *           (decode page, section "gen_mask_tkg": the index < cache length
 *           cut); the current tokens see each other causally.
 *   window  > 0: sliding window as in the prefill predicate; <= 0: none.
 *   part_o  device float [batch, s_active, n_q_heads, max_splits, head_dim],
 *   part_lse device float [batch, s_active, n_q_heads, max_splits]:
 *           caller-owned workspace. Split s of sequence b covers cache
 *           tokens [s*split_len, min(cache_len[b], (s+1)*split_len)). For
 *           every split that starts below cache_len[b], part_o holds the
 *           split's normalised attention output and part_lse its natural-log
 *           log-sum-exp of the scaled visible scores (-inf and zeros if the
 *           split has no visible key). Splits at or beyond cache_len[b] are
 *           not written.
 *   split_len must be a positive multiple of 16 (and of page_size when
 *   paged); max_splits * split_len must cover the longest cache
 *   (>= max_pages_per_seq * page_size when paged); a split may span at most
 *   256 pages (split_len / page_size <= 256, else ATTN_ERR_UNSUPPORTED).
 * Requires head_dim in {64, 128, 256}, dtype f16 or bf16, and
 * (n_q_heads / n_kv_heads) * s_active <= 32 (<= 16 at head_dim 256).
 */
int attn_decode_fwd(const void* q, attn_strides q_st,
                    const void* k_cache, const void* v_cache, attn_strides kv_st,
                    const uint32_t* block_table, int max_pages_per_seq, int page_size,
                    const int32_t* cache_len, attn_dtype dtype, int batch, int s_active,
                    int n_q_heads, int n_kv_heads, int head_dim, float scale, int window,
                    float* part_o, float* part_lse, int split_len, int max_splits,
                    void* hip_stream);

/*
 * attn_decode_fwd for a K/V cache stored in FP8 E4M3 (the OCP "e4m3fn"
 * encoding: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, NaN = S.1111.111, largest value 448) — the decode page's
 * FP8-e4m3 KV cache ("Flash-Attention: Decode (TKG)", section "KV-cache
 * layouts and access", flat cache: the FP8 K path). k_cache and v_cache hold one byte per element with the same
 * layouts and strides (in elements, i.e. bytes) as for attn_decode_fwd; a
 * stored code x stands for k_scale * value(x) (K) or v_scale * value(x) (V).
 * q (`dtype`, f16 or bf16), the workspace and the partials are as for
 * attn_decode_fwd, and attn_decode_combine merges them as usual. The codes
 * are widened exactly to the 16-bit type of q before the products, so the
 * only rounding beyond attn_decode_fwd is the cache's own. k_scale and
 * v_scale must be finite (else ATTN_ERR_INVALID); NaN codes give NaN rows.
 */
int attn_decode_fwd_fp8kv(const void* q, attn_strides q_st,
                          const uint8_t* k_cache, const uint8_t* v_cache, attn_strides kv_st,
                          const uint32_t* block_table, int max_pages_per_seq, int page_size,
                          const int32_t* cache_len, attn_dtype dtype, int batch, int s_active,
                          int n_q_heads, int n_kv_heads, int head_dim, float scale,
                          float k_scale, float v_scale, int window,
                          float* part_o, float* part_lse, int split_len, int max_splits,
                          void* hip_stream);

/*
 * Merge of the split partials written by attn_decode_fwd with the same
 * (cache_len, split_len, max_splits, batch, s_active, n_q_heads, head_dim):
 *   M = max_s lse_s,  w_s = exp(lse_s - M),  O = sum_s w_s O_s / sum_s w_s
 * over the splits that start below cache_len[b] — the cross-section merge
 * O_acc = alpha * O_prev + O_section of the CTE page (section "Algorithm —
 * running-sum update, reciprocal, output accumulate"), generalised to many
 * partials. Rows whose splits are all empty output zeros.
 *   o [batch, s_active, n_q_heads, head_dim] device, `dtype` (f16 or bf16).
 */
int attn_decode_combine(const float* part_o, const float* part_lse, const int32_t* cache_len,
                        int split_len, int max_splits, int batch, int s_active, int n_q_heads,
                        int head_dim, void* o, attn_strides o_st, attn_dtype dtype,
                        void* hip_stream);

/*
 * attn_decode_combine with the same two optional extras as
 * attn_prefill_fwd_ex (NULL = not used):
 *   lse    device float [batch, s_active, n_q_heads]: natural-log
 *          log-sum-exp of each merged row (over all its splits and the sink);
 *   sinks  device float [n_q_heads]: attention sink per q-head, merged as
 *          one more partial whose output is zero and whose log-sum-exp is the
 *          sink.
 * The split kernel is unchanged: the sink enters once per row, here.
 */
int attn_decode_combine_ex(const float* part_o, const float* part_lse, const int32_t* cache_len,
                           int split_len, int max_splits, int batch, int s_active, int n_q_heads,
                           int head_dim, void* o, attn_strides o_st, attn_dtype dtype,
                           float* lse, const float* sinks, void* hip_stream);

/*
 * Device-side check of a page table before attn_decode_fwd /
 * attn_decode_fwd_fp8kv, which trust it: the decode page's gather faults on
 * an out-of-range page index ("Flash-Attention: Decode (TKG)", section
 * "Paged / block cache"). For every sequence b it checks that 0 <=
 * cache_len[b] <= max_pages_per_seq * page_size and that the entries of the
 * pages below ceil(cache_len[b] / page_size) are < num_pages (the pool's
 * page count). result: device int32[2], written on the stream: result[0] =
 * number of problems found, result[1] = the lowest flat index
 * b * max_pages_per_seq + page of one (the first slot of the row for a bad
 * cache_len), or INT32_MAX if none. Reads only the table rows' checked
 * entries and cache_len. Returns ATTN_ERR_INVALID for malformed arguments,
 * ATTN_ERR_UNSUPPORTED when batch * max_pages_per_seq >= 2^31.
 */
int attn_decode_validate_pages(const uint32_t* block_table, int max_pages_per_seq, int page_size,
                               const int32_t* cache_len, int batch, int64_t num_pages, int32_t* result,
                               void* hip_stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): attn_decode_fwd followed by attn_decode_combine in one call,
 * writing o [batch, s_active, n_q_heads, head_dim] (`dtype`, o_st strides)
 * with the same kernels and bit-identical results, but with the split
 * partials in a device array of the library (ATTN_DECODE_NOALLOC_MAX_BYTES
 * per GPU, held until the process ends) instead of a caller's workspace.
 * Arguments are those of attn_decode_fwd (16-bit cache) and
 * attn_decode_combine. The partials need batch * s_active * n_q_heads *
 * max_splits * (head_dim + 1) * 4 bytes; more than the maximum returns
 * ATTN_ERR_UNSUPPORTED before any HIP call (use longer splits, or the
 * workspace entry points). No call allocates, frees or memsets anything; the
 * first call on a device looks up the array's address there (the device of
 * hip_stream must be current). Every call on a GPU shares that GPU's array:
 * calls that overlap on one GPU (concurrent streams or threads) race and
 * must be serialised by the caller.
 */
#define ATTN_DECODE_NOALLOC_MAX_BYTES ((size_t)32 << 20)

int attn_decode_fwd_noalloc(const void* q, attn_strides q_st,
                            const void* k_cache, const void* v_cache, attn_strides kv_st,
                            const uint32_t* block_table, int max_pages_per_seq, int page_size,
                            const int32_t* cache_len, attn_dtype dtype, int batch, int s_active,
                            int n_q_heads, int n_kv_heads, int head_dim, float scale, int window,
                            int split_len, int max_splits, void* o, attn_strides o_st,
                            void* hip_stream);

/* Bytes of part_o and part_lse that attn_decode_fwd needs. Returns ATTN_OK or ATTN_ERR_INVALID. */
int attn_decode_workspace_size(int batch, int s_active, int n_q_heads, int head_dim, int max_splits,
                               size_t* part_o_bytes, size_t* part_lse_bytes);

/* Which kernel the prefill entry points launch for a call of these sizes. It is host
 * arithmetic only (no HIP call, no device memory): the entry points take their launch
 * from this same choice, so a caller or a test can see which kernel a shape exercises.
 * fp8_kv: K/V as FP8 codes (attn_prefill_fwd_fp8kv); packed: cumulative offsets given
 * (attn_prefill_varlen_fwd, whose batch, max_seqlen_q and max_seqlen_kv are then batch,
 * seqlen_q and seqlen_kv here); has_positions: per-row positions given. Returns an
 * attn_prefill_kernel value (> 0), or minus ATTN_ERR_INVALID / ATTN_ERR_UNSUPPORTED for
 * arguments the entry points reject with that status, or 0 for an empty call. */
typedef enum {
    ATTN_PREFILL_F32 = 1,         /* fp32 on the vector ALUs */
    ATTN_PREFILL_MFMA_4W = 2,     /* 16-bit, four waves per 128-row q tile */
    ATTN_PREFILL_MFMA_8W = 3,     /* 16-bit, eight waves per 256-row q tile (wide grids) */
    ATTN_PREFILL_PAIR = 4,        /* head_dim 256, paired waves, one workgroup per q tile */
    ATTN_PREFILL_PAIR_ITEMS = 5,  /* head_dim 256, paired waves, one persistent workgroup per CU */
    ATTN_PREFILL_MFMA_8W_FP8 = 6, /* FP8 K/V staged and widened in LDS, eight waves (wide grids, head_dim 128) */
    ATTN_PREFILL_FP8_4W = 7       /* FP8 K/V widened in registers, four waves */
} attn_prefill_kernel;
int attn_prefill_kernel_for(attn_dtype dtype, int fp8_kv, int packed, int has_positions, int batch,
                            int n_q_heads, int n_kv_heads, int seqlen_q, int seqlen_kv, int head_dim,
                            int causal, int window);
/* Name of an attn_prefill_kernel value ("?" for others). Never NULL. */
const char* attn_prefill_kernel_name(int kernel);
/* Kv-heads per workgroup of the decode split kernel (attn_decode_fwd, _fp8kv) for these
 * sizes: 1, 2, 4 or 8. Host arithmetic only, as above; 0 for sizes it does not cover. */
int attn_decode_heads_per_workgroup(int fp8_kv, int batch, int n_kv_heads, int head_dim, int max_splits);

/* Static description of a status code. Never NULL. */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
