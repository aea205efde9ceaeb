// C ABI of libattn: argument validation, kernel selection, launch.
//
// Every host-checkable precondition is checked before the first HIP call,
// so a rejected call enqueues nothing and leaves no HIP error state. After a
// launch the HIP error state is read (which also clears it) and turned into
// ATTN_ERR_LAUNCH.
#include <cmath>
#include <cstdint>

#include "attn.h"
#include "kernels.hpp"

namespace {

bool supported_head_dim(int d) { return d == 64 || d == 128 || d == 256; }

int elem_bytes(int dtype) { return dtype == ATTN_F32 ? 4 : 2; }

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Optional float arrays (NULL allowed) must be 4-byte aligned.
bool aligned4(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 3u) == 0; }

bool strides_ok(const attn_strides& s, int eb) {
    return s.batch >= 0 && s.seq >= 0 && s.head >= 0 && (s.batch * eb) % 16 == 0 && (s.seq * eb) % 16 == 0 &&
           (s.head * eb) % 16 == 0;
}

attn::Strides3 conv(const attn_strides& s) { return attn::Strides3{s.batch, s.seq, s.head}; }

// Sign flip applied to Q when scale < 0, so kernels only ever see |scale|.
uint32_t q_flip_mask(float scale, int dtype) {
    if (!(scale < 0.f)) return 0u;
    return dtype == ATTN_F32 ? 0x80000000u : 0x80008000u;
}

// |scale| * log2(e), kept at or above `floor` so that a masked score (float32
// min) times it stays far below every real scaled score and below the kernels'
// initial running max (-1e30): its exp2 is then exactly 0 and it never moves
// the max. The 16-bit prefill kernel relies on this arithmetic alone (floor
// 1e-8, which changes the weights by at most |score| * 1e-8 relative for
// smaller scales); the other kernels also zero masked entries explicitly and
// keep the floor at 1e-30, which only separates a zero scale from the mask.
float scaled_log2e(float scale, double floor) {
    const double c = std::fabs((double)scale) * 1.4426950408889634;
    return (float)(c < floor ? floor : c);
}

int status_of(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH; }

}  // namespace

extern "C" {

static_assert((int)ATTN_PREFILL_F32 == attn::kPrefillF32 && (int)ATTN_PREFILL_MFMA_4W == attn::kPrefillMfma4 &&
                  (int)ATTN_PREFILL_MFMA_8W == attn::kPrefillMfma8 && (int)ATTN_PREFILL_PAIR == attn::kPrefillPair &&
                  (int)ATTN_PREFILL_PAIR_ITEMS == attn::kPrefillPairItems &&
                  (int)ATTN_PREFILL_MFMA_8W_FP8 == attn::kPrefillMfma8Kv8 && (int)ATTN_PREFILL_FP8_4W == attn::kPrefillF8kv4,
              "the C ABI's kernel ids are the dispatch's");

int attn_prefill_kernel_for(attn_dtype dtype, int fp8_kv, int packed, int has_positions, int batch,
                            int n_q_heads, int n_kv_heads, int seqlen_q, int seqlen_kv, int head_dim,
                            int causal, int window) {
    // the entry points' checks that depend on these arguments alone (prefill_impl)
    if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return -ATTN_ERR_INVALID;
    if (batch < 0 || n_q_heads < 0 || n_kv_heads < 0 || seqlen_q < 0 || seqlen_kv < 0 || head_dim <= 0)
        return -ATTN_ERR_INVALID;
    if (batch == 0 || n_q_heads == 0 || seqlen_q == 0) return 0;
    if (n_kv_heads == 0 || n_q_heads % n_kv_heads != 0) return -ATTN_ERR_INVALID;
    if (!supported_head_dim(head_dim)) return -ATTN_ERR_UNSUPPORTED;
    if (window > 0 && !causal) return -ATTN_ERR_UNSUPPORTED;
    if (fp8_kv && dtype == ATTN_F32) return -ATTN_ERR_UNSUPPORTED;
    const int w = window > 0 ? window : 0;
    const int mask = !causal ? attn::kMaskNone : (w > 0 ? attn::kMaskCausalWindow : attn::kMaskCausal);
    const attn::PrefillShape sh{(int)dtype, fp8_kv != 0, packed != 0, has_positions != 0, batch, n_q_heads,
                                seqlen_q, seqlen_kv, head_dim, mask, w};
    return attn::prefill_kernel(sh);
}

const char* attn_prefill_kernel_name(int kernel) {
    switch (kernel) {
        case ATTN_PREFILL_F32: return "prefill_f32";
        case ATTN_PREFILL_MFMA_4W: return "prefill_mfma (4 waves)";
        case ATTN_PREFILL_MFMA_8W: return "prefill_mfma (8 waves)";
        case ATTN_PREFILL_PAIR: return "prefill_pair";
        case ATTN_PREFILL_PAIR_ITEMS: return "prefill_pair_items";
        case ATTN_PREFILL_MFMA_8W_FP8: return "prefill_mfma (8 waves, FP8 K/V)";
        case ATTN_PREFILL_FP8_4W: return "prefill_f8kv";
        default: return "?";
    }
}

int attn_decode_heads_per_workgroup(int fp8_kv, int batch, int n_kv_heads, int head_dim, int max_splits) {
    if (batch <= 0 || n_kv_heads <= 0 || max_splits <= 0 || !supported_head_dim(head_dim)) return 0;
    return attn::decode_heads_per_workgroup(fp8_kv != 0, head_dim, n_kv_heads, batch, max_splits);
}

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_INVALID: return "invalid argument";
        case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
        case ATTN_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

}  // extern "C"

namespace {
// Shared by the prefill entry points. With cu_seqlens_q != NULL the sequences
// are packed (seqlen_q / seqlen_kv are then the largest lengths and the batch
// strides are not used).
int prefill_impl(const void* q, attn_strides q_st, const void* k, attn_strides k_st, const void* v,
                 attn_strides v_st, void* o, attn_strides o_st, attn_dtype dtype, int batch, int n_q_heads,
                 int n_kv_heads, int seqlen_q, int seqlen_kv, int head_dim, float scale, int causal, int window,
                 float* lse, const float* sinks, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                 const int32_t* positions, void* hip_stream, int kv_bytes = 0, float v_scale = 1.f) {
    if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_INVALID;
    if (batch < 0 || n_q_heads < 0 || n_kv_heads < 0 || seqlen_q < 0 || seqlen_kv < 0 || head_dim <= 0)
        return ATTN_ERR_INVALID;
    if (!std::isfinite(scale)) return ATTN_ERR_INVALID;
    if (batch == 0 || n_q_heads == 0 || seqlen_q == 0) return ATTN_OK;
    if (n_kv_heads == 0 || n_q_heads % n_kv_heads != 0) return ATTN_ERR_INVALID;
    if (!supported_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED;
    if (window > 0 && !causal) return ATTN_ERR_UNSUPPORTED;
    const int eb = elem_bytes(dtype);
    const bool fp8 = kv_bytes == 1;  // K and V hold FP8 E4M3 codes (strides in bytes)
    if (fp8 && dtype == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
    const int kvb = fp8 ? 1 : eb;
    if (!q || !o || !aligned16(q) || !aligned16(o)) return ATTN_ERR_INVALID;
    if (seqlen_kv > 0 && (!k || !v || !aligned16(k) || !aligned16(v))) return ATTN_ERR_INVALID;
    if (!strides_ok(q_st, eb) || !strides_ok(k_st, kvb) || !strides_ok(v_st, kvb) || !strides_ok(o_st, eb))
        return ATTN_ERR_INVALID;
    if (!aligned4(lse) || !aligned4(sinks)) return ATTN_ERR_INVALID;
    if ((cu_seqlens_q == nullptr) != (cu_seqlens_kv == nullptr)) return ATTN_ERR_INVALID;
    if (cu_seqlens_q && (!aligned4(cu_seqlens_q) || !aligned4(cu_seqlens_kv))) return ATTN_ERR_INVALID;
    if (!aligned4(positions)) return ATTN_ERR_INVALID;
    // byte offsets inside one 64-row K/V tile (buffer records and lane offsets) are kept in 31 bits
    if ((k_st.seq * 64 + head_dim) * kvb >= ((int64_t)1 << 31) || (v_st.seq * 64 + head_dim) * kvb >= ((int64_t)1 << 31))
        return ATTN_ERR_UNSUPPORTED;
    const int64_t tiles = (seqlen_q + 63) / 64;
    if (tiles * batch * n_q_heads >= (int64_t)1 << 31) return ATTN_ERR_UNSUPPORTED;

    attn::PrefillParams p{};
    p.q = q; p.k = k; p.v = v; p.o = o;
    p.qs = conv(q_st); p.ks = conv(k_st); p.vs = conv(v_st); p.os = conv(o_st);
    p.batch = batch; p.n_q_heads = n_q_heads; p.n_kv_heads = n_kv_heads; p.group = n_q_heads / n_kv_heads;
    p.seqlen_q = seqlen_q; p.seqlen_kv = seqlen_kv;
    p.window = window > 0 ? window : 0;
    p.c = scaled_log2e(scale, dtype == ATTN_F32 ? 1e-30 : 1e-8);
    p.qflip = q_flip_mask(scale, dtype);
    p.lse = lse;
    p.sinks = sinks;
    p.cu_seqlens_q = cu_seqlens_q;
    p.cu_seqlens_kv = cu_seqlens_kv;
    p.positions = positions;
    // Deal workgroups to XCDs in chunks of the q-heads sharing a kv-head: in one
    // fixed order when every (sequence, kv-head) then stays on one XCD (1), and in
    // rounds of alternating XCD order on the eight-wave grids (the same rule as the
    // prefill dispatch's) whose q-heads share kv-heads (2).
    p.xcd_chunks = ((int64_t)batch * n_kv_heads) % 8 == 0 ? 1
                   : (!cu_seqlens_q && head_dim <= 128 && n_q_heads / n_kv_heads >= 2 &&
                      (int64_t)((seqlen_q + 255) / 256) * batch * n_q_heads >= 512) ? 2 : 0;
    p.v_scale = v_scale;
    const int mask = !causal ? attn::kMaskNone : (p.window > 0 ? attn::kMaskCausalWindow : attn::kMaskCausal);
    if (fp8) return status_of(attn::launch_prefill_f8kv(p, (int)dtype, head_dim, mask, (hipStream_t)hip_stream));
    return status_of(attn::launch_prefill(p, (int)dtype, head_dim, mask, (hipStream_t)hip_stream));
}
}  // namespace

extern "C" {

int attn_prefill_fwd_ex(const void* q, attn_strides q_st, const void* k, attn_strides k_st, const void* v,
                        attn_strides v_st, void* o, attn_strides o_st, attn_dtype dtype, int batch, int n_q_heads,
                        int n_kv_heads, int seqlen_q, int seqlen_kv, int head_dim, float scale, int causal,
                        int window, float* lse, const float* sinks, void* hip_stream) {
    return prefill_impl(q, q_st, k, k_st, v, v_st, o, o_st, dtype, batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_kv,
                        head_dim, scale, causal, window, lse, sinks, nullptr, nullptr, nullptr, hip_stream);
}

int attn_prefill_fwd_fp8kv(const void* q, attn_strides q_st, const uint8_t* k, attn_strides k_st, const uint8_t* v,
                           attn_strides v_st, void* o, attn_strides o_st, attn_dtype dtype, int batch, int n_q_heads,
                           int n_kv_heads, int seqlen_q, int seqlen_kv, int head_dim, float scale, float k_scale,
                           float v_scale, int causal, int window, float* lse, const float* sinks, void* hip_stream) {
    if (!std::isfinite(k_scale) || !std::isfinite(v_scale) || !std::isfinite(scale * k_scale))
        return ATTN_ERR_INVALID;
    return prefill_impl(q, q_st, k, k_st, v, v_st, o, o_st, dtype, batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_kv,
                        head_dim, scale * k_scale, causal, window, lse, sinks, nullptr, nullptr, nullptr, hip_stream,
                        1, v_scale);
}

int attn_prefill_varlen_fwd(const void* q, attn_strides q_st, const void* k, attn_strides k_st, const void* v,
                            attn_strides v_st, void* o, attn_strides o_st, attn_dtype dtype, int batch,
                            int n_q_heads, int n_kv_heads, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_kv, int max_seqlen_q, int max_seqlen_kv, int head_dim,
                            float scale, int causal, int window, float* lse, const float* sinks,
                            const int32_t* positions, void* hip_stream) {
    if (batch > 0 && (!cu_seqlens_q || !cu_seqlens_kv)) return ATTN_ERR_INVALID;
    return prefill_impl(q, q_st, k, k_st, v, v_st, o, o_st, dtype, batch, n_q_heads, n_kv_heads, max_seqlen_q,
                        max_seqlen_kv, head_dim, scale, causal, window, lse, sinks, cu_seqlens_q, cu_seqlens_kv,
                        positions, hip_stream);
}

int attn_prefill_fwd(const void* q, attn_strides q_st, const void* k, attn_strides k_st, const void* v,
                     attn_strides v_st, void* o, attn_strides o_st, attn_dtype dtype, int batch, int n_q_heads,
                     int n_kv_heads, int seqlen_q, int seqlen_kv, int head_dim, float scale, int causal, int window,
                     void* hip_stream) {
    return attn_prefill_fwd_ex(q, q_st, k, k_st, v, v_st, o, o_st, dtype, batch, n_q_heads, n_kv_heads, seqlen_q,
                               seqlen_kv, head_dim, scale, causal, window, nullptr, nullptr, hip_stream);
}

int attn_decode_validate_pages(const uint32_t* block_table, int max_pages_per_seq, int page_size,
                               const int32_t* cache_len, int batch, int64_t num_pages, int32_t* result,
                               void* hip_stream) {
    if (batch < 0 || max_pages_per_seq < 0 || page_size <= 0 || num_pages < 0) return ATTN_ERR_INVALID;
    if (!result || !aligned4(result)) return ATTN_ERR_INVALID;
    if (batch > 0 && (!block_table || !cache_len || max_pages_per_seq == 0)) return ATTN_ERR_INVALID;
    if (!aligned4(block_table) || !aligned4(cache_len)) return ATTN_ERR_INVALID;
    if ((int64_t)batch * max_pages_per_seq >= ((int64_t)1 << 31)) return ATTN_ERR_UNSUPPORTED;
    return status_of(attn::launch_validate_pages(block_table, cache_len, batch, max_pages_per_seq, page_size,
                                                 num_pages, result, (hipStream_t)hip_stream));
}

int attn_decode_workspace_size(int batch, int s_active, int n_q_heads, int head_dim, int max_splits,
                               size_t* part_o_bytes, size_t* part_lse_bytes) {
    if (batch < 0 || s_active < 0 || n_q_heads < 0 || head_dim < 0 || max_splits < 0) return ATTN_ERR_INVALID;
    const size_t rows = (size_t)batch * (size_t)s_active * (size_t)n_q_heads * (size_t)max_splits;
    if (part_o_bytes) *part_o_bytes = rows * (size_t)head_dim * sizeof(float);
    if (part_lse_bytes) *part_lse_bytes = rows * sizeof(float);
    return ATTN_OK;
}

namespace {
// Validation and parameters shared by attn_decode_fwd, attn_decode_fwd_fp8kv
// and attn_decode_fwd_noalloc (kv_bytes is the cache's element size). Sets
// `empty` for a problem with nothing to compute. With workspace = false the
// partials' pointers are not checked (the caller supplies them later).
int decode_setup(const void* q, attn_strides q_st, const void* k_cache, const void* v_cache, attn_strides kv_st,
                 const uint32_t* block_table, int max_pages_per_seq, int page_size, const int32_t* cache_len,
                 attn_dtype dtype, int batch, int s_active, int n_q_heads, int n_kv_heads, int head_dim, float scale,
                 int window, float* part_o, float* part_lse, int split_len, int max_splits, int kv_bytes,
                 float v_scale, bool workspace, attn::DecodeParams& p, bool& empty) {
    empty = false;
    if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_INVALID;
    if (batch < 0 || s_active < 0 || n_q_heads < 0 || n_kv_heads < 0 || head_dim <= 0) return ATTN_ERR_INVALID;
    if (!std::isfinite(scale)) return ATTN_ERR_INVALID;
    if (batch == 0 || s_active == 0 || n_q_heads == 0) {
        empty = true;
        return ATTN_OK;
    }
    if (n_kv_heads == 0 || n_q_heads % n_kv_heads != 0) return ATTN_ERR_INVALID;
    if (split_len <= 0 || split_len % 16 != 0 || max_splits <= 0) return ATTN_ERR_INVALID;
    if (block_table) {
        if (page_size <= 0 || max_pages_per_seq <= 0 || split_len % page_size != 0) return ATTN_ERR_INVALID;
        if ((int64_t)max_splits * split_len < (int64_t)max_pages_per_seq * page_size) return ATTN_ERR_INVALID;
        if (split_len / page_size > attn::kDecodeMaxSplitPages) return ATTN_ERR_UNSUPPORTED;
    }
    if (dtype == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
    if (!supported_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED;
    if ((int64_t)(n_q_heads / n_kv_heads) * s_active > (head_dim <= 128 ? 32 : 16)) return ATTN_ERR_UNSUPPORTED;
    if (max_splits > 65535 || batch > 65535) return ATTN_ERR_UNSUPPORTED;
    const int eb = elem_bytes(dtype);
    if (!q || !k_cache || !v_cache || !cache_len) return ATTN_ERR_INVALID;
    if (workspace && (!part_o || !part_lse || !aligned16(part_o))) return ATTN_ERR_INVALID;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return ATTN_ERR_INVALID;
    if (!strides_ok(q_st, eb) || !strides_ok(kv_st, kv_bytes)) return ATTN_ERR_INVALID;

    p = attn::DecodeParams{};
    p.q = q; p.k = k_cache; p.v = v_cache;
    p.qs = conv(q_st); p.kvs = conv(kv_st);
    p.block_table = block_table; p.cache_len = cache_len;
    p.part_o = part_o; p.part_lse = part_lse;
    p.batch = batch; p.s_active = s_active; p.n_q_heads = n_q_heads; p.n_kv_heads = n_kv_heads;
    p.group = n_q_heads / n_kv_heads;
    p.max_pages_per_seq = block_table ? max_pages_per_seq : 0;
    p.page_size = block_table ? page_size : 1;
    p.page_shift = -1;
    for (int sh = 0; sh < 31; ++sh)
        if ((1 << sh) == p.page_size) p.page_shift = sh;
    p.window = window > 0 ? window : 0;
    p.split_len = split_len; p.max_splits = max_splits;
    p.c = scaled_log2e(scale, 1e-30);
    p.qflip = q_flip_mask(scale, dtype);
    p.kv_fp8 = kv_bytes == 1;
    p.v_scale = v_scale;
    p.lane_addr32 = (int64_t)16 * (kv_st.seq + head_dim) * kv_bytes < ((int64_t)1 << 31);
    return ATTN_OK;
}

int decode_fwd_impl(const void* q, attn_strides q_st, const void* k_cache, const void* v_cache, attn_strides kv_st,
                    const uint32_t* block_table, int max_pages_per_seq, int page_size, const int32_t* cache_len,
                    attn_dtype dtype, int batch, int s_active, int n_q_heads, int n_kv_heads, int head_dim,
                    float scale, int window, float* part_o, float* part_lse, int split_len, int max_splits,
                    int kv_bytes, float v_scale, void* hip_stream) {
    attn::DecodeParams p;
    bool empty;
    const int st = decode_setup(q, q_st, k_cache, v_cache, kv_st, block_table, max_pages_per_seq, page_size, cache_len,
                                dtype, batch, s_active, n_q_heads, n_kv_heads, head_dim, scale, window, part_o,
                                part_lse, split_len, max_splits, kv_bytes, v_scale, true, p, empty);
    if (st != ATTN_OK || empty) return st;
    return status_of(attn::launch_decode(p, (int)dtype, head_dim, (hipStream_t)hip_stream));
}

// Validation and parameters of the combine (shared by attn_decode_combine_ex
// and attn_decode_fwd_noalloc); the partials' pointers are checked by the caller.
int combine_setup(const int32_t* cache_len, int split_len, int max_splits, int batch, int s_active, int n_q_heads,
                  int head_dim, void* o, attn_strides o_st, attn_dtype dtype, float* lse, const float* sinks,
                  attn::CombineParams& p, bool& empty) {
    empty = false;
    if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_INVALID;
    if (batch < 0 || s_active < 0 || n_q_heads < 0 || head_dim <= 0) return ATTN_ERR_INVALID;
    if (batch == 0 || s_active == 0 || n_q_heads == 0) {
        empty = true;
        return ATTN_OK;
    }
    if (split_len <= 0 || max_splits <= 0) return ATTN_ERR_INVALID;
    if (dtype == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
    if (!supported_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED;
    if ((int64_t)batch * s_active * n_q_heads >= (int64_t)1 << 31) return ATTN_ERR_UNSUPPORTED;
    if (!cache_len || !o || !aligned16(o)) return ATTN_ERR_INVALID;
    if (!strides_ok(o_st, elem_bytes(dtype))) return ATTN_ERR_INVALID;
    if (!aligned4(lse) || !aligned4(sinks)) return ATTN_ERR_INVALID;

    p = attn::CombineParams{};
    p.cache_len = cache_len; p.o = o; p.os = conv(o_st);
    p.batch = batch; p.s_active = s_active; p.n_q_heads = n_q_heads;
    p.split_len = split_len; p.max_splits = max_splits;
    p.lse = lse; p.sinks = sinks;
    return ATTN_OK;
}
}  // namespace

int attn_decode_fwd(const void* q, attn_strides q_st, const void* k_cache, const void* v_cache, attn_strides kv_st,
                    const uint32_t* block_table, int max_pages_per_seq, int page_size, const int32_t* cache_len,
                    attn_dtype dtype, int batch, int s_active, int n_q_heads, int n_kv_heads, int head_dim,
                    float scale, int window, float* part_o, float* part_lse, int split_len, int max_splits,
                    void* hip_stream) {
    return decode_fwd_impl(q, q_st, k_cache, v_cache, kv_st, block_table, max_pages_per_seq, page_size, cache_len,
                           dtype, batch, s_active, n_q_heads, n_kv_heads, head_dim, scale, window, part_o, part_lse,
                           split_len, max_splits, elem_bytes(dtype), 1.f, hip_stream);
}

int attn_decode_fwd_fp8kv(const void* q, attn_strides q_st, const uint8_t* k_cache, const uint8_t* v_cache,
                          attn_strides kv_st, const uint32_t* block_table, int max_pages_per_seq, int page_size,
                          const int32_t* cache_len, attn_dtype dtype, int batch, int s_active, int n_q_heads,
                          int n_kv_heads, int head_dim, float scale, float k_scale, float v_scale, int window,
                          float* part_o, float* part_lse, int split_len, int max_splits, void* hip_stream) {
    if (!std::isfinite(k_scale) || !std::isfinite(v_scale) || !std::isfinite(scale * k_scale))
        return ATTN_ERR_INVALID;
    return decode_fwd_impl(q, q_st, k_cache, v_cache, kv_st, block_table, max_pages_per_seq, page_size, cache_len,
                           dtype, batch, s_active, n_q_heads, n_kv_heads, head_dim, scale * k_scale, window, part_o,
                           part_lse, split_len, max_splits, 1, v_scale, hip_stream);
}

int attn_decode_combine_ex(const float* part_o, const float* part_lse, const int32_t* cache_len, int split_len,
                           int max_splits, int batch, int s_active, int n_q_heads, int head_dim, void* o,
                           attn_strides o_st, attn_dtype dtype, float* lse, const float* sinks, void* hip_stream) {
    attn::CombineParams p;
    bool empty;
    const int st = combine_setup(cache_len, split_len, max_splits, batch, s_active, n_q_heads, head_dim, o, o_st,
                                 dtype, lse, sinks, p, empty);
    if (st != ATTN_OK || empty) return st;
    if (!part_o || !part_lse) return ATTN_ERR_INVALID;
    p.part_o = part_o; p.part_lse = part_lse;
    return status_of(attn::launch_combine(p, (int)dtype, head_dim, (hipStream_t)hip_stream));
}

int attn_decode_combine(const float* part_o, const float* part_lse, const int32_t* cache_len, int split_len,
                        int max_splits, int batch, int s_active, int n_q_heads, int head_dim, void* o,
                        attn_strides o_st, attn_dtype dtype, void* hip_stream) {
    return attn_decode_combine_ex(part_o, part_lse, cache_len, split_len, max_splits, batch, s_active, n_q_heads,
                                  head_dim, o, o_st, dtype, nullptr, nullptr, hip_stream);
}

int attn_decode_fwd_noalloc(const void* q, attn_strides q_st, const void* k_cache, const void* v_cache,
                            attn_strides kv_st, const uint32_t* block_table, int max_pages_per_seq, int page_size,
                            const int32_t* cache_len, attn_dtype dtype, int batch, int s_active, int n_q_heads,
                            int n_kv_heads, int head_dim, float scale, int window, int split_len, int max_splits,
                            void* o, attn_strides o_st, void* hip_stream) {
    attn::DecodeParams dp;
    attn::CombineParams cp;
    bool empty;
    int st = decode_setup(q, q_st, k_cache, v_cache, kv_st, block_table, max_pages_per_seq, page_size, cache_len,
                          dtype, batch, s_active, n_q_heads, n_kv_heads, head_dim, scale, window, nullptr, nullptr,
                          split_len, max_splits, elem_bytes(dtype), 1.f, false, dp, empty);
    if (st != ATTN_OK || empty) return st;
    st = combine_setup(cache_len, split_len, max_splits, batch, s_active, n_q_heads, head_dim, o, o_st, dtype,
                       nullptr, nullptr, cp, empty);
    if (st != ATTN_OK || empty) return st;
    // the partials, [rows, max_splits, head_dim] then [rows, max_splits] f32, must fit the device array
    const uint64_t slots = (uint64_t)batch * (uint64_t)s_active * (uint64_t)n_q_heads * (uint64_t)max_splits;
    if (slots * ((uint64_t)head_dim + 1) * sizeof(float) > ATTN_DECODE_NOALLOC_MAX_BYTES) return ATTN_ERR_UNSUPPORTED;
    void* scratch = nullptr;
    if (attn::decode_scratch(&scratch) != hipSuccess) return ATTN_ERR_LAUNCH;
    float* const part_o = (float*)scratch;
    float* const part_lse = part_o + slots * (uint64_t)head_dim;
    dp.part_o = part_o;
    dp.part_lse = part_lse;
    cp.part_o = part_o;
    cp.part_lse = part_lse;
    const hipStream_t s = (hipStream_t)hip_stream;
    st = status_of(attn::launch_decode(dp, (int)dtype, head_dim, s));
    if (st != ATTN_OK) return st;
    return status_of(attn::launch_combine(cp, (int)dtype, head_dim, s));
}

}  // extern "C"
