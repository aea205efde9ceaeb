// Kernel parameter blocks and launchers (internal to libattn; the public
// interface is include/attn.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct Strides3 {
    int64_t batch, seq, head;
};

struct PrefillParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    Strides3 qs, ks, vs, os;
    int batch, n_q_heads, n_kv_heads, group;  // group = n_q_heads / n_kv_heads
    int seqlen_q, seqlen_kv;                   // per sequence, or the largest ones with cu_seqlens_*
    int window;                                // > 0 only together with causal
    int n_q_tiles;
    float c;          // |scale| * log2(e): scores are kept in scaled log2 units
    uint32_t qflip;   // 0x80008000 (16-bit) / 0x80000000 (f32) flips Q's sign when scale < 0
    float* lse;           // NULL, or [batch, seqlen_q, n_q_heads] natural-log log-sum-exp per row
    const float* sinks;   // NULL, or [n_q_heads] sink logits (scaled-score units)
    // NULL, or packed sequences: [batch + 1] cumulative row offsets; sequence b
    // owns q/o rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) and k/v rows
    // [cu_seqlens_kv[b], cu_seqlens_kv[b+1]) (batch strides unused; lse is [total_q, n_q_heads])
    const int32_t* cu_seqlens_q;
    const int32_t* cu_seqlens_kv;
    // NULL, or the position of every query row ([batch * seqlen_q] or [total_q], the
    // lse row order); key j is visible to a row at position P iff j <= P (causal)
    // and j >= P - window + 1. Nondecreasing within a sequence.
    const int32_t* positions;
    // Deal workgroups to XCDs in kv-head groups: 0 no, 1 in one order (batch * n_kv_heads
    // % 8 == 0: each K/V stream on one XCD), 2 in rounds of alternating XCD order.
    int xcd_chunks;
    float v_scale;    // FP8 K/V (prefill_f8kv): V row = v_scale * its codes (K's scale is folded into c)
};

struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    Strides3 qs, kvs;
    const uint32_t* block_table;  // NULL -> flat cache
    const int32_t* cache_len;
    float* part_o;
    float* part_lse;
    int batch, s_active, n_q_heads, n_kv_heads, group;
    int max_pages_per_seq, page_size, page_shift;
    int window, split_len, max_splits;
    float c;
    uint32_t qflip;
    int kv_fp8;       // the cache holds FP8 E4M3 codes (decode_split_f8)
    float v_scale;    // FP8 caches: V row = v_scale * its codes (K's scale is folded into c)
    int lane_addr32;  // the byte offset of row 15 of a 16-row group, plus a head row, fits 31 bits
};

struct CombineParams {
    const float* part_o;
    const float* part_lse;
    const int32_t* cache_len;
    void* o;
    Strides3 os;
    int batch, s_active, n_q_heads, split_len, max_splits;
    float* lse;           // NULL, or [batch, s_active, n_q_heads] natural-log log-sum-exp per row
    const float* sinks;   // NULL, or [n_q_heads] sink logits (scaled-score units)
};

// Largest number of pages one decode split may span (split_len / page_size).
constexpr int kDecodeMaxSplitPages = 256;

enum MaskMode { kMaskNone = 0, kMaskCausal = 1, kMaskCausalWindow = 2 };
enum DType { kF32 = 0, kF16 = 1, kBF16 = 2 };

// The kernel a prefill call launches, chosen from its sizes and flags alone
// (host code; the launch functions below dispatch on this same choice).
enum PrefillKernel {
    kPrefillF32 = 1,        // prefill_f32
    kPrefillMfma4 = 2,      // prefill_mfma, four waves (128 rows)
    kPrefillMfma8 = 3,      // prefill_mfma, eight waves (256 rows)
    kPrefillPair = 4,       // prefill_pair (D = 256), one workgroup per q tile
    kPrefillPairItems = 5,  // prefill_pair_items (D = 256), persistent
    kPrefillMfma8Kv8 = 6,   // prefill_mfma, eight waves, FP8 K/V staging
    kPrefillF8kv4 = 7,      // prefill_f8kv, four waves
};
struct PrefillShape {
    int dtype;
    bool fp8, packed, positions;  // FP8 K/V codes; cu_seqlens given; per-row positions given
    int batch, n_q_heads, seqlen_q, seqlen_kv, head_dim, mask, window;
};
int prefill_kernel(const PrefillShape& s);
// Kv-heads (waves) per workgroup of the decode split kernel for these sizes.
int decode_heads_per_workgroup(bool fp8, int head_dim, int n_kv_heads, int batch, int max_splits);

// Each returns the hipError_t of its launch (hipSuccess on success).
hipError_t launch_prefill(const PrefillParams& p, int dtype, int head_dim, int mask, hipStream_t s);
// K and V as FP8 E4M3 codes (k/v strides in bytes); dtype (f16/bf16) is Q's and O's.
hipError_t launch_prefill_f8kv(const PrefillParams& p, int dtype, int head_dim, int mask, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int dtype, int head_dim, hipStream_t s);
hipError_t launch_combine(const CombineParams& p, int dtype, int head_dim, hipStream_t s);
// Device address of the allocation-free decode's partials on the current
// device (ATTN_DECODE_NOALLOC_MAX_BYTES, looked up once per device).
hipError_t decode_scratch(void** addr);
hipError_t launch_validate_pages(const uint32_t* block_table, const int32_t* cache_len, int batch,
                                 int max_pages_per_seq, int page_size, int64_t num_pages, int32_t* result,
                                 hipStream_t s);

}  // namespace attn
