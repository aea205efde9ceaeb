// Prefill (context) flash-attention forward for gfx950.
//
// f16 / bf16: prefill_mfma — one workgroup per (128-row Q tile, q-head,
// batch), four waves of 32 query rows each. Q stays in VGPRs as MFMA
// operands for the whole kernel ("Q resident, KV streams": CTE page,
// section "Tile shapes and residency"); 64-key K/V tiles stream through LDS
// in two buffers each, filled by buffer loads that write LDS directly. Each
// wave computes the transposed score tile S^T = K Q^T with
// v_mfma_f32_32x32x16, so every lane owns one query row and the row max /
// row sum are in-lane plus one v_permlane32_swap. The f32 S^T accumulator
// layout is exactly the B-operand layout of O^T += V^T P^T, so P never
// leaves registers; V^T is read from the row-major V tile with
// ds_read_b64_tr_b16. O^T (f32) and m, l stay in VGPRs. The key loop is
// software-pipelined: the QK MFMAs of tile j+1 run while the VALU
// exponentiates tile j.
//
// Online softmax per tile (CTE page, "The online-softmax recurrence"; minfer
// 8n page, section 2.1): scores are kept in scaled log2 units t = s*scale*log2e,
//   m_new = max(m, max_j t_j),  alpha = 2^(m - m_new),  p_j = 2^(t_j - m_new),
//   l = alpha*l + sum_j p_j,     O = alpha*O + P V,       finally O * (1/l).
// m starts at a finite sentinel so alpha is 0 on first contact and never NaN
// (optimum-neuron guide, "Numerical stability"); an all-masked row ends with
// l = 0 and is written as zeros (minfer 8n page, the epilogue).
//
// Masking (CTE page, "Algorithm — compute-skip" and the affine_select
// masks): tiles that no row of the wave can see are skipped, tiles that all
// rows see entirely take no per-element mask, and only the tiles that
// straddle the diagonal, the window edge or the end of K are masked.
//
// f32: prefill_f32 — the same recurrence on the vector ALUs (no f32 MFMA
// shortcut is used): 64 rows per workgroup, four lanes per row.
//
// FP8 K/V: K and V stored as E4M3 codes, widened exactly into the same LDS
// tiles. On the wide grids that take eight waves (D = 128) prefill_mfma
// itself stages the codes (KV8) and keeps its whole pipeline; elsewhere
// prefill_f8kv runs prefill_mfma's per-tile math without the pipeline.
#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {

template <bool B>
struct BoolC {
    static constexpr bool value = B;
};

constexpr int PF_ROWS_PER_WAVE = 32;  // query rows per wave
constexpr int PF_BN = 64;   // keys per tile

// LDS layout of the K and V tiles: row-major, 16-byte chunk c of row r stored
// at chunk c ^ f(r). Tiles are filled with direct-to-LDS loads (each 1 KB load
// covers whole rows), so bank conflicts are avoided by swizzling, not padding.
// K: a 16-lane group of a b128 read hits rows r..r+15 at one chunk.
template <int D>
__device__ __forceinline__ int pf_kswz(int row) {
    return D == 64 ? ((row >> 1) & 7) : (row & 15);
}
// V: 32 lanes of a transpose read hit rows R..R+3 (R % 4 == 0) at four adjacent chunks.
template <int D>
__device__ __forceinline__ int pf_vswz(int row) {
    return D == 64 ? 4 * ((row >> 1) & 1) : 4 * (row & 3);
}

// Q fragments of one lane (B operand of S^T = K Q^T: row l32, d = 16s + 8hf
// .. +8), read from qrow (already offset by 8 hf), which must point at a row
// of the sequence (callers clamp it); the fragments are zeros when the lane's
// own row is outside the sequence (valid = false). The loads are unconditional
// and the zeroing is a mask applied afterwards, so no branch separates the
// loads and nothing waits for them before the caller's next loads are issued.
// qflip flips the sign bits when the scale is negative.
template <int D>
__device__ __forceinline__ void pf_load_q(s16x8 (&qf)[D / 16], const uint16_t* qrow, bool valid, uint32_t qflip) {
    const uint32_t keep = valid ? 0xffffffffu : 0u;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        uint4 x = *(const uint4*)(qrow + 16 * s);
        x.x = (x.x & keep) ^ qflip; x.y = (x.y & keep) ^ qflip;
        x.z = (x.z & keep) ^ qflip; x.w = (x.w & keep) ^ qflip;
        qf[s] = __builtin_bit_cast(s16x8, x);
    }
}

// The same in two parts, for a caller that issues the loads, then more loads,
// and applies the mask only after a wait that covers them: the raw fragments,
// then the mask and the sign flip. (pf_load_q's loads and masks in one place
// can be compiled as a load, a wait and a mask per fragment.)
template <int D>
__device__ __forceinline__ void pf_load_q_raw(uint4 (&x)[D / 16], const uint16_t* qrow) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) x[s] = *(const uint4*)(qrow + 16 * s);
}
template <int D>
__device__ __forceinline__ void pf_mask_q(s16x8 (&qf)[D / 16], const uint4 (&x)[D / 16], bool valid, uint32_t qflip) {
    const uint32_t keep = valid ? 0xffffffffu : 0u;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        uint4 y = x[s];
        y.x = (y.x & keep) ^ qflip; y.y = (y.y & keep) ^ qflip;
        y.z = (y.z & keep) ^ qflip; y.w = (y.w & keep) ^ qflip;
        qf[s] = __builtin_bit_cast(s16x8, y);
    }
}

// One lane's half of an output row, each value multiplied by inv and rounded
// (NaN throughout when nan_row: a NaN or +inf sink). O^T tile dt holds
// d = 32 dt + 8 rq + 4 hf .. +4 in registers 4 rq .. 4 rq + 3; the two lanes
// that share a row (hf = 0, 1) swap halves with v_permlane32_swap, so that per
// d tile and pair of 8-dim groups (2p, 2p + 1) lane hf holds dims
// 32 dt + 8 (2p + hf) .. +8 and writes them as one 16-byte store: each row gets
// 32 contiguous bytes per store instruction (8-byte stores of each lane's own
// groups measured 8% slower on the D = 256 window workload). Called by the
// whole wave (the swaps need both halves); `store` says whether this lane's
// row is written (the same for both lanes of a row).
template <bool BF16, int NDT>
__device__ __forceinline__ void pf_store_o16(const f32x16 (&o)[NDT], float inv, uint16_t* orow, int hf, bool nan_row,
                                             bool store) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            // packed pairs of 8-dim groups 2pp (this lane's dims 4 hf .. +4) and 2pp + 1
            uint32_t a[2], b[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                a[e] = pack2_16<BF16>(o[dt][8 * pp + 2 * e] * inv, o[dt][8 * pp + 2 * e + 1] * inv);
                b[e] = pack2_16<BF16>(o[dt][8 * pp + 4 + 2 * e] * inv, o[dt][8 * pp + 4 + 2 * e + 1] * inv);
            }
            uint32_t w0[2], w1[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const auto r = __builtin_amdgcn_permlane32_swap(a[e], b[e], false, false);
                w0[e] = r[0];  // hf = 0: its own group 2pp; hf = 1: the other lane's group 2pp + 1
                w1[e] = r[1];  // hf = 0: the other lane's group 2pp; hf = 1: its own group 2pp + 1
            }
            uint4 pk = make_uint4(w0[0], w0[1], w1[0], w1[1]);
            if (nan_row) pk = make_uint4(kNaN16x2<BF16>, kNaN16x2<BF16>, kNaN16x2<BF16>, kNaN16x2<BF16>);
            if (store) *(uint4*)(orow + 32 * dt + 8 * (2 * pp + hf)) = pk;
        }
}

// The row's log-sum-exp (natural log) from m and l in scaled log2 units: -inf
// without any visible key or sink, NaN bits with a NaN or +inf sink.
__device__ __forceinline__ void pf_store_lse(float* dst, float m, float l, bool nan_row) {
    const uint32_t bits = nan_row ? kNaN32
                                  : __float_as_uint(l > 0.f ? (m + __log2f(l)) * 0.69314718055994531f : -__builtin_inff());
    *(uint32_t*)dst = bits;
}

// 16 FP8 E4M3 codes -> two 16-byte chunks of 16-bit floats (codes 0..7, 8..15),
// widened exactly (gfx950's v_cvt_scalef32_pk_*_fp8 with scale 1: every E4M3
// value is representable in bf16 and f16).
template <bool BF16>
__device__ __forceinline__ void widen_e4m3x16(uint4 x, uint4& lo, uint4& hi) {
    uint32_t wv[8];
    const uint32_t src[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (BF16) {
            wv[2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src[e], 1.0f, false));
            wv[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src[e], 1.0f, true));
        } else {
            wv[2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src[e], 1.0f, false));
            wv[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src[e], 1.0f, true));
        }
    }
    lo = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    hi = make_uint4(wv[4], wv[5], wv[6], wv[7]);
}

// NW waves per workgroup: 4 (two workgroups per CU for D <= 128) or 8 (one
// workgroup per CU, twice the query rows per K/V tile: half the L2-to-LDS
// traffic per FLOP).
//
// KV8: K and V hold FP8 E4M3 codes with one scale per tensor (a code stands
// for scale times its value; the host folds K's scale into c, V's scale
// multiplies the output) -- the decode page's quantised cache read by a
// prefill. Eight waves and D = 128 only. The codes of each tile go HBM->LDS
// into a staging area with the same direct loads, each wave's load to its own
// kilobyte (8 rows); at the end of the step before the tile is needed the
// same wave widens them (exactly) and writes them into the 16-bit tile layout
// below, and the end-of-step barrier publishes them. A wave only reads back
// what its own load wrote, so the staging needs no barrier of its own, and
// the 16-bit tiles, the fragment reads and all of the math are the 16-bit
// path's.
template <bool BF16, int D, int MASK, int NW, bool KV8 = false>
__global__ __launch_bounds__(64 * NW, (NW == 8 ? 1 : 2)) void prefill_mfma(PrefillParams p) {
    static_assert(D == 64 || D == 128, "head_dim 256 takes prefill_pair / prefill_pair_items");
    static_assert(!KV8 || (NW == 8 && D == 128), "FP8 K/V: eight waves, D = 128");
    constexpr int PF_BM = PF_ROWS_PER_WAVE * NW;  // query rows per workgroup
    constexpr int PF_THREADS = 64 * NW;
    constexpr int CPR = D / 8;              // 16-byte chunks per row
    constexpr int TILE = PF_BN * D;         // elements of one K or V tile
    constexpr int LPW = TILE / 512 / NW;    // 1 KB direct loads per wave per tile
    static_assert(LPW >= 1, "every wave loads part of each tile");
    constexpr int NDT = D / 32;             // 32-wide d tiles of O^T
    // K and V tiles, separate objects so waits on one buffer's refill never
    // cover reads of the other: three K buffers (one barrier per key tile),
    // and three V buffers for eight waves (whose one workgroup per CU has the
    // LDS for them), two for four (80 KB at D = 128: two workgroups per CU).
    constexpr int NB = NW == 8 ? 3 : 2;                  // V buffers
    __shared__ __attribute__((aligned(16))) uint16_t Ks0[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Ks1[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Ks2[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vs0[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vs1[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vs2[NB == 3 ? TILE : 8];
    // FP8 staging: two tiles of codes per tensor (separate objects, as above)
    constexpr int TILE8 = KV8 ? TILE : 16;
    __shared__ __attribute__((aligned(16))) uint8_t Sk0[TILE8];
    __shared__ __attribute__((aligned(16))) uint8_t Sk1[TILE8];
    __shared__ __attribute__((aligned(16))) uint8_t Sv0[TILE8];
    __shared__ __attribute__((aligned(16))) uint8_t Sv1[TILE8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int l32 = lane & 31;
    const int hf = lane >> 5;   // wave half
    const int g = lane >> 4;    // 16-lane group
    const int r16 = lane & 15;

    // Workgroup -> (q tile, batch, q-head). In the logical order, consecutive
    // workgroups are the heads of one q tile and causal tiles come heaviest
    // first. The hardware deals workgroups to the 8 XCDs round robin
    // (workgroup i to XCD i % 8) and each XCD has its own L2. With
    // p.xcd_chunks the logical order is dealt out in chunks of `group`
    // workgroups — the q-heads that share one kv-head — with a whole chunk on
    // one XCD. Mode 1 (batch * n_kv_heads a multiple of 8): all chunks of one
    // (sequence, kv-head) then land on the same XCD, so each K/V stream is
    // fetched into one L2 only (measured 8% faster on 16 packed prompts).
    // Mode 2 (eight-wave grids whose q-heads share kv-heads, fewer than 8
    // streams): the heads of one q tile then share one L2, and successive
    // rounds of chunks are dealt in opposite XCD order, so that with causal
    // tiles (heaviest first) every XCD gets the same work (32K causal, 8
    // q-heads over 1 kv-head: 2% faster together with the three-buffer
    // pipeline). Mode 1 keeps one order, which alternating would break. The
    // last partial round keeps the plain order.
    const int nbh = p.batch * p.n_q_heads;
    int wid = (int)blockIdx.x;
    if (p.xcd_chunks) {
        const int G = p.group, round = 8 * G;
        const int full = ((int)gridDim.x / round) * round;
        if (wid < full) {
            const int xcd = wid & 7, k = wid >> 3, r = k / G;
            wid = (r * 8 + ((p.xcd_chunks == 2 && (r & 1)) ? 7 - xcd : xcd)) * G + k % G;
        }
    }
    // A grid that fits on the chip in one go (256 < workgroups <= 512, two
    // per CU) has no later workgroups to fill in behind the heavy ones, so
    // its second half runs lightest first: the CU that starts a heavy tile
    // is then paired with a light one (2K causal, 28 heads: 4% faster).
    if constexpr (NW == 4 && D <= 128) {
        const int n = (int)gridDim.x;
        if (n > 256 && n <= 512 && wid >= 256) wid = 256 + (n - 1 - wid);
    }
    const int qt = p.n_q_tiles - 1 - wid / nbh;
    const int bh = wid % nbh;
    const int b = bh / p.n_q_heads;
    const int h = bh % p.n_q_heads;
    const int hk = h / p.group;

    // Sequence b's sizes and the element offsets of its first rows: sequences
    // of one fixed size, or packed sequences delimited by cumulative offsets.
    int sq = p.seqlen_q, skv = p.seqlen_kv;
    int64_t q_at = (int64_t)b * p.qs.batch, k_at = (int64_t)b * p.ks.batch, v_at = (int64_t)b * p.vs.batch,
            o_at = (int64_t)b * p.os.batch, lse_at = (int64_t)b * p.seqlen_q;
    if (p.cu_seqlens_q) {
        const int qs0 = p.cu_seqlens_q[b], ks0 = p.cu_seqlens_kv[b];
        sq = min(p.cu_seqlens_q[b + 1] - qs0, p.seqlen_q);
        skv = p.cu_seqlens_kv[b + 1] - ks0;
        q_at = (int64_t)qs0 * p.qs.seq;
        o_at = (int64_t)qs0 * p.os.seq;
        lse_at = qs0;
        k_at = (int64_t)ks0 * p.ks.seq;
        v_at = (int64_t)ks0 * p.vs.seq;
    }
    const int off = skv - sq;  // query row i sits at position i + off

    const int q0 = qt * PF_BM;
    if (q0 >= sq) return;  // a tile past this sequence's end (packed sequences only)
    const int qlast = min(q0 + PF_BM, sq) - 1;
    // Position of query row i: i + off (bottom-right alignment), or the caller's
    // positions of packed rows (nondecreasing within a sequence).
    auto pos_of = [&](int i) -> int { return p.positions ? p.positions[lse_at + min(i, sq - 1)] : i + off; };
    int kv_lo = 0, kv_hi = skv;
    if (MASK >= kMaskCausal) kv_hi = min(kv_hi, pos_of(qlast) + 1);
    if (MASK == kMaskCausalWindow) kv_lo = max(0, pos_of(q0) - p.window + 1);
    const int j_begin = kv_lo / PF_BN;
    const int j_end = kv_hi > kv_lo ? (kv_hi + PF_BN - 1) / PF_BN : j_begin;

    const int wq0 = q0 + 32 * w;                   // first row of this wave
    const int wq1 = min(wq0 + 31, sq - 1); // last valid row of this wave
    const bool wave_live = wq0 < sq;
    const int my_q = wq0 + l32;                    // the query row this lane owns
    const int my_pos = pos_of(my_q);
    const int wpos0 = pos_of(wq0), wpos1 = pos_of(wq1);  // positions of the wave's first and last rows

    // Q stays in VGPRs; it is loaded in the prologue, after the first K/V
    // tiles have been requested, so that both latencies overlap.
    s16x8 qf[D / 16];
    const uint16_t* qrow = (const uint16_t*)p.q + q_at + (int64_t)min(my_q, sq - 1) * p.qs.seq +
                           (int64_t)h * p.qs.head + 8 * hf;

    const uint16_t* kbase = (const uint16_t*)p.k + k_at + (int64_t)hk * p.ks.head;
    const uint16_t* vbase = (const uint16_t*)p.v + v_at + (int64_t)hk * p.vs.head;
    // Tile rows outside [kv_lo, seqlen_kv) are loaded as copies of the nearest
    // valid row: they are masked out (probability exactly 0) and no memory
    // outside the visible key range is touched. Every load is unconditional.
    const int key_min = kv_lo, key_max = skv - 1;
    // Tiles are filled with buffer loads straight into LDS: the tile's first
    // row is the buffer base (a uniform descriptor), lane offsets are 32-bit
    // byte offsets. Direct load i (0 <= i < TILE/512) covers tile rows RPL*i
    // .. RPL*i + RPL-1; lane l takes row RPL*i + l/CPR and the swizzled chunk
    // (l%CPR ^ g(l/CPR)) ^ U(i) (the K or V swizzle factored into a lane part
    // and a uniform part), so a lane keeps two offsets per tensor. A tile
    // spans fewer than 64 * seq + D elements, whose bytes the host keeps below 2^31.
    // Edge tiles clamp row by row.
    constexpr int RPL = 64 / CPR;
    const int lrow = lane / CPR, lcs = lane % CPR;
    const uint32_t kx = 16u * (uint32_t)(lcs ^ (D == 64 ? lrow >> 1 : lrow));
    const uint32_t vx = 16u * (uint32_t)(lcs ^ (D == 64 ? 4 * ((lrow >> 1) & 1) : 4 * lrow));
    const uint32_t kl = 2u * (uint32_t)lrow * (uint32_t)p.ks.seq, vl = 2u * (uint32_t)lrow * (uint32_t)p.vs.seq;
    // (Two plain lambdas rather than one generic one: a generic lambda here
    // keeps the compiler's host pass from emitting the kernel's launch stub.)
    auto load_tile_impl = [&](uint16_t* dst, const uint16_t* base, int64_t seq, int j, uint32_t lane_row_off,
                              uint32_t lane_chunk_off, bool is_k) __attribute__((always_inline)) {
        const int kv0 = j * PF_BN;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)kv0 * seq), (short)0, 0x7fffffff, 0x00020000);
        if (kv0 >= key_min && kv0 + PF_BN - 1 <= key_max) {
#pragma unroll
            for (int ii = 0; ii < LPW; ++ii) {
                const int i = w * LPW + ii;
                const uint32_t u = is_k ? (D == 64 ? (4 * i) & 7 : (4 * i) & 15) : 0;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 512 * i), 16,
                                                         lane_row_off + (lane_chunk_off ^ (16u * u)),
                                                         (uint32_t)(2 * RPL * i) * (uint32_t)seq, 0, 0);
            }
        } else {
            // Rare path: recomputed on each use (the opaque copy keeps the
            // compiler from hoisting per-load lane values out of the loop).
            int lr = lrow;
            asm volatile("" : "+v"(lr));
#pragma unroll
            for (int ii = 0; ii < LPW; ++ii) {
                const int i = w * LPW + ii;
                const int row = RPL * i + lr, cs = lcs;
                const int key = min(max(kv0 + row, key_min), key_max);  // kv0 <= key <= kv0 + 63
                const int c = cs ^ (is_k ? pf_kswz<D>(row) : pf_vswz<D>(row));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 512 * i), 16,
                                                         2u * ((uint32_t)(key - kv0) * (uint32_t)seq + 8u * c), 0, 0, 0);
            }
        }
    };
    auto load_k_tile = [&](uint16_t* dst, int j) __attribute__((always_inline)) { load_tile_impl(dst, kbase, p.ks.seq, j, kl, kx, true); };
    auto load_v_tile = [&](uint16_t* dst, int j) __attribute__((always_inline)) { load_tile_impl(dst, vbase, p.vs.seq, j, vl, vx, false); };
    // In-loop loads: one direct load at a time, so that they can be spread
    // over the MFMA stages. Tiles past the first one lie above kv_lo, so only
    // their end can leave the visible range; the descriptor's record count
    // stops at the end of row key_max and the range check drops the rows past
    // it (their LDS rows keep zeros or an earlier tile's finite rows, which
    // are masked). Each load's row offset is in its own lane offset register
    // (computed once), so the range check covers the whole offset.
    uint32_t kvo[LPW], vvo[LPW];
#pragma unroll
    for (int ii = 0; ii < (KV8 ? 0 : LPW); ++ii) {
        const int i = w * LPW + ii;
        const uint32_t uk = D == 64 ? (4 * i) & 7 : (4 * i) & 15;
        const uint32_t uv = 0;
        uint32_t ko = kl + (kx ^ (16u * uk)) + (uint32_t)(2 * RPL * i) * (uint32_t)p.ks.seq;
        uint32_t vo = vl + (vx ^ (16u * uv)) + (uint32_t)(2 * RPL * i) * (uint32_t)p.vs.seq;
        asm volatile("" : "+v"(ko), "+v"(vo));
        kvo[ii] = ko;
        vvo[ii] = vo;
    }
    auto tile_rsrc = [&](const uint16_t* base, int64_t seq, int j) __attribute__((always_inline)) {
        const int kv0 = j * PF_BN;
        const uint32_t nrec =
            kv0 + PF_BN - 1 <= key_max ? 0x7fffffffu : 2u * ((uint32_t)(key_max - kv0) * (uint32_t)seq + (uint32_t)D);
        return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)kv0 * seq), (short)0, nrec, 0x00020000);
    };
    auto load_part = [&](uint16_t* dst, __amdgpu_buffer_rsrc_t rs, uint32_t voff, int ii) __attribute__((always_inline)) {
        const int i = w * LPW + ii;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 512 * i), 16, voff, 0, 0, 0);
    };

    // FP8 codes (KV8): one direct load per wave, tensor and tile; lane
    // c8 = 64 w + lane takes codes 16 (c8 % 8) .. +16 of tile row c8 / 8 into
    // staging bytes 16 c8 .. +16, so wave w's kilobyte holds rows 8w .. 8w + 7.
    // The wave widens them in another order: lane l takes codes
    // 8 (l % 16) .. +8 of rows 8w + l / 16 and 8w + 4 + l / 16, so the 16 lanes
    // of each 16-byte store write the 16 chunks of one row (16 distinct bank
    // groups; the load order, two adjacent chunks of two rows per 16 lanes, put
    // two lanes on each even group of the V tile). Range-limited loads of the
    // last tile drop the rows past key_max, whose staging bytes keep the codes
    // of an earlier tile (visible keys: finite), masked like every row past
    // the end.
    const int c8 = 64 * w + lane, row8 = c8 >> 3, col8 = 16 * (c8 & 7);
    const uint8_t* const kbase8 = (const uint8_t*)p.k + k_at + (int64_t)hk * p.ks.head;
    const uint8_t* const vbase8 = (const uint8_t*)p.v + v_at + (int64_t)hk * p.vs.head;
    uint32_t k8o = 0, v8o = 0;
    if constexpr (KV8) {
        k8o = (uint32_t)row8 * (uint32_t)p.ks.seq + (uint32_t)col8;
        v8o = (uint32_t)row8 * (uint32_t)p.vs.seq + (uint32_t)col8;
        asm volatile("" : "+v"(k8o), "+v"(v8o));
    }
    auto tile_rsrc8 = [&](const uint8_t* base, int64_t seq, int j) __attribute__((always_inline)) {
        const int kv0 = j * PF_BN;
        const uint32_t nrec =
            kv0 + PF_BN - 1 <= key_max ? 0x7fffffffu : (uint32_t)(key_max - kv0) * (uint32_t)seq + (uint32_t)D;
        return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)kv0 * seq), (short)0, nrec, 0x00020000);
    };
    auto stage_part = [&](uint8_t* dst, __amdgpu_buffer_rsrc_t rs, uint32_t voff) __attribute__((always_inline)) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 1024 * w), 16, voff, 0, 0, 0);
    };
    // A whole tile with its rows clamped one by one into [key_min, key_max] (the prologue's tiles).
    auto stage_clamped = [&](uint8_t* dst, const uint8_t* base, int64_t seq, int j) __attribute__((always_inline)) {
        const int kv0 = j * PF_BN;
        const int key = min(max(kv0 + row8, key_min), key_max);  // kv0 <= key <= kv0 + 63
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)kv0 * seq), (short)0, 0x7fffffff, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 1024 * w), 16,
                                                 (uint32_t)(key - kv0) * (uint32_t)seq + (uint32_t)col8, 0, 0, 0);
    };
    const int wr0 = 8 * w + (lane >> 4), wch = lane & 15;
    auto stage_read = [&](const uint8_t* src) __attribute__((always_inline)) {
        const uint8_t* b0 = src + 1024 * w + 128 * (lane >> 4) + 8 * wch;
        const uint2 a = *(const uint2*)b0, b = *(const uint2*)(b0 + 512);
        return make_uint4(a.x, a.y, b.x, b.y);
    };
    auto widen_store = [&](uint16_t* dst, uint4 x, bool is_k) __attribute__((always_inline)) {
        uint4 lo, hi;
        widen_e4m3x16<BF16>(x, lo, hi);
        const int r1 = wr0 + 4;
        const int s0 = is_k ? pf_kswz<D>(wr0) : pf_vswz<D>(wr0);
        const int s1 = is_k ? pf_kswz<D>(r1) : pf_vswz<D>(r1);
        *(uint4*)((char*)dst + wr0 * D * 2 + 16 * (wch ^ s0)) = lo;
        *(uint4*)((char*)dst + r1 * D * 2 + 16 * (wch ^ s1)) = hi;
    };
    auto widen_tile = [&](uint16_t* dst, const uint8_t* src, bool is_k) __attribute__((always_inline)) {
        widen_store(dst, stage_read(src), is_k);
    };

    // Running max in scaled log2 units. It only moves when a row's tile max
    // exceeds it by more than kLazyRescale, so O and l are rescaled rarely;
    // in between, probabilities are at most 2^kLazyRescale (the result is the
    // same softmax for any m >= the true running max minus that margin).
    constexpr float kLazyRescale = 8.0f;
    float m_i = kMaxInit, l_i = 0.f;
    f32x16 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16{};
    const uint32_t one2 = BF16 ? 0x3F803F80u : 0x3C003C00u;  // two 16-bit 1.0s for the row-sum dot2

    auto tile_empty = [&](int j) __attribute__((always_inline)) {
        const int kv0 = j * PF_BN;
        bool e = !wave_live || j >= j_end;
        if (MASK >= kMaskCausal) e |= kv0 > wpos1;
        if (MASK == kMaskCausalWindow) e |= kv0 + PF_BN - 1 < wpos0 - p.window + 1;
        return e;
    };
    auto tile_full = [&](int j) __attribute__((always_inline)) {
        const int kv0 = j * PF_BN;
        bool f = kv0 + PF_BN <= skv;
        if (MASK >= kMaskCausal) f &= kv0 + PF_BN - 1 <= wpos0;
        if (MASK == kMaskCausalWindow) f &= kv0 >= wpos1 - p.window + 1;
        return f;
    };

    // LDS byte offsets of the MFMA fragments. The swizzled chunk of a K
    // fragment is (2s + hf) ^ kswz(row) = 2s ^ (hf ^ kswz(row)), and kswz is
    // the same for rows l32 and 32 + l32, so fragment s of the first block
    // sits at kfrag ^ 32s and the second block 64*D bytes further. A V^T
    // fragment of d tile dt sits at vfrag ^ 64dt plus a row offset that is a
    // compile-time constant (vswz depends on the row only through row % 4 for
    // D >= 128 and (row / 2) % 2 for D = 64, which the u and +8 row steps
    // leave unchanged). Every fragment offset is computed once and kept in
    // its own register (made opaque so the compiler cannot recompute it in
    // the loop); the buffer and row steps are constants folded into the LDS
    // instructions' offset fields.
    const uint32_t kfrag = (uint32_t)(l32 * D * 2) | (16u * (uint32_t)(hf ^ pf_kswz<D>(l32)));
    const int vr0 = 4 * hf + (r16 >> 2);                  // V^T row of this lane in chunk 0
    const int vcl = 2 * (g & 1) + ((r16 & 3) >> 1);       // chunk within a 32-wide d tile
    const uint32_t vfrag = (uint32_t)(vr0 * D * 2) | (16u * (uint32_t)(vcl ^ pf_vswz<D>(vr0))) | (8u * (r16 & 1));
    auto opaque = [](uint32_t x) __attribute__((always_inline)) {
        asm volatile("" : "+v"(x));
        return x;
    };
    auto lds_frag8 = [](const uint16_t* base, uint32_t byte_off) __attribute__((always_inline)) {
        return *(const s16x8*)((const char*)base + byte_off);
    };
    constexpr int NS = D / 16;          // K chunks of 16 along d
    uint32_t koff[NS], voff[NDT];       // per-fragment offset registers
#pragma unroll
    for (int s = 0; s < NS; ++s) koff[s] = opaque(kfrag ^ (32u * s));
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) voff[dt] = opaque(vfrag ^ (64u * dt));

    // S^T of one 64-key tile: two 32-key blocks x 32 queries; lane holds keys
    // 32t + 8(r/4) + 4hf + r%4 of its query row in register r of block t.
    // The two blocks' MFMA chains are interleaved.
    auto qk_tile = [&](f32x16& s0, f32x16& s1, const uint16_t* Kt) __attribute__((always_inline)) {
        const uint32_t kf = opaque(kfrag);
        s0 = f32x16{};
        s1 = f32x16{};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const uint32_t off = kf ^ (32u * s);
            const s16x8 a0 = lds_frag8(Kt, off);
            const s16x8 a1 = lds_frag8(Kt + 32 * D, off);
            s0 = mfma32x32x16<BF16>(a0, qf[s], s0);
            s1 = mfma32x32x16<BF16>(a1, qf[s], s1);
        }
    };
    // This lane's visible keys form one range [key_lo, key_lo + key_span]
    // (span < 0: none), so each score takes one unsigned compare: key - key_lo
    // in [0, span].
    int key_hi = skv - 1, key_lo = 0;
    if (MASK >= kMaskCausal) key_hi = min(key_hi, my_pos);
    if (MASK == kMaskCausalWindow) key_lo = max(key_lo, my_pos - p.window + 1);
    const bool none_visible = key_hi < key_lo;
    const uint32_t key_span = none_visible ? 0u : (uint32_t)(key_hi - key_lo);
    if (none_visible) key_lo = INT_MIN / 2;  // no key of any tile lies at key_lo + [0, 0]
    auto mask_half = [&](f32x16& sacc, int kv0, int t) __attribute__((always_inline)) {
        const int base = kv0 + 32 * t + 4 * hf - key_lo;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const uint32_t d = (uint32_t)(base + 8 * (r >> 2) + (r & 3));
            sacc[r] = d <= key_span ? sacc[r] : kMaskedScore;
        }
    };
    // Row max of a tile (raw scores), combined over the two lane halves.
    auto max_tile = [&](const f32x16& s0, const f32x16& s1) __attribute__((always_inline)) {
        float mx = kMaskedScore;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = max3f(mx, s0[r], s1[r]);
        return max_with_other_half(mx);
    };
    // Move m (and rescale O and l) for rows whose tile max passed m + margin.
    // A row that sees no key of the tile has max = the mask value, and
    // mask * c is far below any m, so such a row keeps its m.
    auto rescale = [&](float mx) __attribute__((always_inline)) {
        const float m_cand = mx * p.c;
        const bool grow = m_cand > m_i + kLazyRescale;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = grow ? m_cand : m_i;
            const float alpha = fast_exp2(m_i - m_new);
            m_i = m_new;
            l_i *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
        }
    };

    // Software pipeline over key tiles, two tiles of scores in registers:
    // step j runs the QK MFMAs of tile j+1 while the VALU turns three quarters
    // of the scores of tile j into probabilities (with the m settled at the
    // end of step j-1), then the P V MFMAs of tile j, ordered by key chunk,
    // while the VALU finishes the last quarter (used by the last chunk's
    // MFMAs) and takes the raw row max of tile j+1; then it sums P(j) and
    // settles m for tile j+1 (rescaling O, which by then includes tile j).
    // The split keeps the VALU work of each half within what runs beside
    // its MFMAs, whichever half the other wave of the SIMD is in. At four
    // waves all of tile j's probabilities are made in the QK part instead
    // (PQ = 16; 2.6% faster on the 2K prefill, whose heavy tiles run without
    // a second wave on their SIMD; eight waves measured 0.5% slower so).
    //
    // Every step runs the same code. A tile that is not fully visible to all
    // rows of the wave gets its hidden scores replaced by the mask value, whose
    // probability is exactly 0 and which never moves m (the host keeps
    // p.c >= 1e-8, so mask * c lies far below the initial m); this covers the
    // diagonal and window-edge tiles, the ragged end of K, tiles past the
    // wave's last visible key, and the tile after the last one (a repeat of
    // the last tile, never used).
    // The step body is laid out by hand in stages separated by scheduling
    // fences: stage s of the QK part issues the two MFMAs of K chunk s, the
    // LDS reads of chunk s+KPD and its share of the probabilities; stage i of
    // the P V part issues MFMA i, the transpose reads of MFMA i+VPRE and its
    // share of the remaining probabilities and of the raw row max of tile
    // j+1. LDS reads thus run at least 128 MFMA cycles ahead of their use:
    // KPD = 2 stages and VPRE = 4 MFMAs at eight waves; at four waves, whose
    // heavy causal tiles often run alone on their SIMD (their partner
    // workgroup done), 3 stages and 6 MFMAs (1-2% faster on the 2K prefill and
    // the packed prompts, same bits; the eight-wave kernel measured no
    // change). The row sums of P(j) (v_dot2c, which stalls when mixed with
    // MFMAs) come after the last MFMA, in two independent chains.
    //
    // Loads and barriers (three K buffers, one barrier per step, at its end):
    // step j issues K(j+3) in its P V part, into the buffer of K(j), which no
    // wave has read since step j-1. With three V buffers it issues V(j+2) at
    // its start and the barrier publishes K(j+2) and V(j+1); with two (four
    // waves) it issues V(j+1) at its start, into the buffer of V(j-1), and the
    // barrier publishes K(j+2) and that V(j+1). Tile indices past the last
    // tile are clamped to it, so every step issues the same loads and each
    // wait is a fixed count: loads complete in issue order, and the barrier
    // waits with vmcnt = the loads issued after the one it needs.
    constexpr int NPV = 4 * NDT;        // P V MFMAs per tile
    constexpr int VPRE = NW == 4 ? 6 : 4;  // P V MFMAs whose fragments are in flight (see above)
    constexpr int PQ = NW == 4 ? 16 : 12;  // probability pairs (of 16) made in the QK part
    constexpr int NPV_EARLY = NPV - NDT;  // P V MFMAs before the last key chunk's
    static_assert(NS >= 4, "the V prefetch is issued in the last two QK stages");
    const int j_last = j_end - 1;
    // KV8 (three buffers): step j stages the codes of V(j+2) (into Svb) and
    // K(j+3) (into Skb) where the 16-bit path loads those tiles, and widens
    // V(j+1) (from Sva) in its QK part and K(j+2) (from Ska) in its P V part,
    // both staged in step j-1, into the third V and K buffers V3, K3, which no
    // wave has read since step j-2; the end-of-step barrier then publishes
    // them as it publishes the direct loads of the 16-bit path. Loads complete
    // in issue order (V(j+1), K(j+2), V(j+2), K(j+3)), so each widening waits
    // with vmcnt = the two loads issued after the one it reads. The codes are
    // read three MFMA stages before they are widened and written (QK stages 2
    // and 5, P V MFMAs 4 and 8: measured best of five placements on the 32K
    // causal workload: 3% faster than widening both at the end of the step).
    auto step = [&](int j, f32x16& c0, f32x16& c1, f32x16& n0, f32x16& n1, uint16_t* Kn, uint16_t* Kl, uint16_t* Vc,
                    uint16_t* Vl, uint16_t* K3, uint16_t* V3, uint8_t* Ska, uint8_t* Skb, uint8_t* Sva,
                    uint8_t* Svb) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t vrs = tile_rsrc(vbase, p.vs.seq, min(j + NB - 1, j_last));
        s16x8 ka[NS][2];
        s16x8 vb[NPV];
        uint32_t pk[16];
        uint4 x8;  // KV8: one lane's staged codes between their read and their widening
        auto kread = [&](int s) __attribute__((always_inline)) {
            ka[s][0] = lds_frag8(Kn, koff[s]);
            ka[s][1] = lds_frag8(Kn + 32 * D, koff[s]);
        };
        auto vread = [&](int i) __attribute__((always_inline)) {
            const int u = i / NDT, dt = i % NDT;
            const char* vb0 = (const char*)Vc + voff[dt];
            vb[i] = concat4(lds_read_tr16((const uint16_t*)(vb0 + 2 * D * (16 * u))),
                            lds_read_tr16((const uint16_t*)(vb0 + 2 * D * (16 * u + 8))));
        };
        // probabilities pk[i] from scores 2(i%8), 2(i%8)+1 of block i/8 of the current tile
        const float neg_m = -m_i;
        auto prob_pair = [&](int i) __attribute__((always_inline)) {
            const f32x16& sc = i < 8 ? c0 : c1;
            const int r = 2 * (i % 8);
            pk[i] = pack2_16<BF16>(fast_exp2(fmaf(sc[r], p.c, neg_m)), fast_exp2(fmaf(sc[r + 1], p.c, neg_m)));
            asm volatile("" ::"v"(pk[i]));  // computed here, not sunk into a later stage
        };
        constexpr int KPD = NW == 4 ? 3 : 2;  // QK stages whose K fragments are in flight
#pragma unroll
        for (int s = 0; s < KPD; ++s) kread(s);
        sched_fence();
        n0 = f32x16{};
        n1 = f32x16{};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            n0 = mfma32x32x16<BF16>(ka[s][0], qf[s], n0);
            n1 = mfma32x32x16<BF16>(ka[s][1], qf[s], n1);
            if constexpr (KV8) {
                if (s == 0) stage_part(Svb, tile_rsrc8(vbase8, p.vs.seq, min(j + 2, j_last)), v8o);
                if (s == 2) {
                    wait_vmcnt<2>();  // V(j+1) in
                    x8 = stage_read(Sva);
                }
                if (s == 5) widen_store(V3, x8, false);
            } else if (s % (NS / LPW) == 0) {
                load_part(Vl, vrs, vvo[s / (NS / LPW)], s / (NS / LPW));
            }
            if (s + KPD < NS) kread(s + KPD);
#pragma unroll
            for (int i = s * PQ / NS; i < (s + 1) * PQ / NS; ++i) prob_pair(i);
            sched_fence();
        }
        const __amdgpu_buffer_rsrc_t krs = tile_rsrc(kbase, p.ks.seq, min(j + 3, j_last));
#pragma unroll
        for (int i = 0; i < VPRE; ++i) vread(i);
        sched_fence();
        // Eight waves: raised wave priority over the P V part, so that a SIMD's
        // arbiter favours the wave feeding O over the other wave's score part
        // (0.9% faster on the 32K causal workload and its FP8-K/V launch, same
        // bits, in interleaved runs of both orders; at four waves it measured
        // slower on the packed prompts, and the paired D = 256 kernel no faster).
        if constexpr (NW == 8) __builtin_amdgcn_s_setprio(1);
        float mx = kMaskedScore;
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            const int u = i / NDT, dt = i % NDT;
            const s16x8 pb = __builtin_bit_cast(s16x8, make_uint4(pk[4 * u], pk[4 * u + 1], pk[4 * u + 2], pk[4 * u + 3]));
            o[dt] = mfma32x32x16<BF16>(vb[i], pb, o[dt]);
            if constexpr (KV8) {
                if (i == 0) stage_part(Skb, tile_rsrc8(kbase8, p.ks.seq, min(j + 3, j_last)), k8o);
                if (i == 4) {
                    wait_vmcnt<2>();  // K(j+2) in
                    x8 = stage_read(Ska);
                }
                if (i == 8) widen_store(K3, x8, true);
            } else if (i % (NPV / LPW) == 0) {
                load_part(Kl, krs, kvo[i / (NPV / LPW)], i / (NPV / LPW));
            }
            if (i + VPRE < NPV) vread(i + VPRE);
            if (i < NPV_EARLY) {
#pragma unroll
                for (int e = PQ + i * (16 - PQ) / NPV_EARLY; e < PQ + (i + 1) * (16 - PQ) / NPV_EARLY; ++e) prob_pair(e);
            }
#pragma unroll
            for (int e = i * 16 / NPV; e < (i + 1) * 16 / NPV; ++e) mx = max3f(mx, n0[e], n1[e]);
            sched_fence();
        }
        if constexpr (NW == 8) __builtin_amdgcn_s_setprio(0);
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            ps0 = dot2_16<BF16>(pk[e], one2, ps0);
            ps1 = dot2_16<BF16>(pk[e + 1], one2, ps1);
        }
        l_i += ps0 + ps1;
        mx = max_with_other_half(mx);
        if (!(wave_live && tile_full(j + 1))) {
            mask_half(n0, (j + 1) * PF_BN, 0);
            mask_half(n1, (j + 1) * PF_BN, 1);
            mx = fminf(mx, max_tile(n0, n1));  // masking only lowers the max
        }
        rescale(mx);
        // K(j+2) in (and V(j+1) with two V buffers and three K buffers:
        // only K(j+3) may still be in flight); every wave is past its reads of V(j).
        if constexpr (!KV8) wait_vmcnt<(NB == 2 ? 1 : 2) * LPW>();
        barrier_lds();
    };

    // Prologue: K(j_begin), V(j_begin), K(j_begin + 1) in, S(j_begin) and its
    // m, then K(j_begin + 2) requested into the buffer of K(j_begin).
    f32x16 sa0, sa1, sb0, sb1;
    const int nt = j_end - j_begin;
    if (nt > 0) {
        if constexpr (KV8) {
            stage_clamped(Sk0, kbase8, p.ks.seq, j_begin);
            stage_clamped(Sv0, vbase8, p.vs.seq, j_begin);
            stage_clamped(Sk1, kbase8, p.ks.seq, min(j_begin + 1, j_last));
            pf_load_q<D>(qf, qrow, my_q < sq, p.qflip);
            wait_vmcnt<0>();
            widen_tile(Ks0, Sk0, true);
            widen_tile(Vs0, Sv0, false);
            widen_tile(Ks1, Sk1, true);
        } else {
            // The first refill of a V buffer in the loop may be range-limited: start it from zeros.
            uint16_t* const vz = NB == 3 ? Vs2 : Vs1;
#pragma unroll
            for (int c = tid; c < TILE / 8; c += PF_THREADS) *(uint4*)(vz + 8 * c) = make_uint4(0, 0, 0, 0);
            // K(j_begin) and Q first: the first scores wait for those only, while
            // V(j_begin) and K(j_begin + 1) arrive behind them.
            load_k_tile(Ks0, j_begin);
            pf_load_q<D>(qf, qrow, my_q < sq, p.qflip);
            if constexpr (NB == 2) {
                load_k_tile(Ks1, min(j_begin + 1, j_last));
                load_v_tile(Vs0, j_begin);
            } else {
                load_v_tile(Vs0, j_begin);
                load_k_tile(Ks1, min(j_begin + 1, j_last));
            }
            wait_vmcnt<2 * LPW>();
        }
        barrier_lds();
        qk_tile(sa0, sa1, Ks0);
        if (!(wave_live && tile_full(j_begin))) {
            mask_half(sa0, j_begin * PF_BN, 0);
            mask_half(sa1, j_begin * PF_BN, 1);
        }
        rescale(max_tile(sa0, sa1));
        if constexpr (!KV8) {
            // K(j_begin + 1) and V(j_begin) in; every wave is past its reads of K(j_begin)
            wait_vmcnt<0>();
            barrier_lds();
        }
        if constexpr (KV8) {
            // codes of V(j_begin + 1) and K(j_begin + 2) (in the loop's order), widened in the first step
            stage_clamped(Sv1, vbase8, p.vs.seq, min(j_begin + 1, j_last));
            stage_clamped(Sk0, kbase8, p.ks.seq, min(j_begin + 2, j_last));
        } else if constexpr (NB == 3) {
            // K(j_begin + 2) and V(j_begin + 1) into buffers no wave has read yet
            load_k_tile(Ks2, min(j_begin + 2, j_last));
            load_v_tile(Vs1, min(j_begin + 1, j_last));
        } else {
            // K(j_begin + 2) into the third K buffer; V(j_begin + 1) is step 0's load
            load_k_tile(Ks2, min(j_begin + 2, j_last));
        }
    }
    if constexpr (NB == 3) {
        // Step r = j - j_begin: K(j+1) sits in buffer (r+1)%3, V(j) in buffer
        // r%3; the step refills K buffer r%3 with K(j+3) and V buffer (r+2)%3
        // with V(j+2). Unrolled by six (the buffers cycle by three, the score
        // registers by two) so that every LDS access names its buffer.
        // KV8 staging cycles by two: even steps widen from Sk0 / Sv1 and stage
        // into Sk1 / Sv0, odd steps the other way round.
        for (int r = 0; r < nt; r += 6) {
            step(j_begin + r, sa0, sa1, sb0, sb1, Ks1, Ks0, Vs0, Vs2, Ks2, Vs1, Sk0, Sk1, Sv1, Sv0);
            if (r + 1 < nt) step(j_begin + r + 1, sb0, sb1, sa0, sa1, Ks2, Ks1, Vs1, Vs0, Ks0, Vs2, Sk1, Sk0, Sv0, Sv1);
            if (r + 2 < nt) step(j_begin + r + 2, sa0, sa1, sb0, sb1, Ks0, Ks2, Vs2, Vs1, Ks1, Vs0, Sk0, Sk1, Sv1, Sv0);
            if (r + 3 < nt) step(j_begin + r + 3, sb0, sb1, sa0, sa1, Ks1, Ks0, Vs0, Vs2, Ks2, Vs1, Sk1, Sk0, Sv0, Sv1);
            if (r + 4 < nt) step(j_begin + r + 4, sa0, sa1, sb0, sb1, Ks2, Ks1, Vs1, Vs0, Ks0, Vs2, Sk0, Sk1, Sv1, Sv0);
            if (r + 5 < nt) step(j_begin + r + 5, sb0, sb1, sa0, sa1, Ks0, Ks2, Vs2, Vs1, Ks1, Vs0, Sk1, Sk0, Sv0, Sv1);
        }
    } else {
        // Three K buffers, two V buffers (four waves): step r reads K(j+1) from
        // K buffer (r+1)%3 and V(j) from V buffer r%2, refills K buffer r%3 with
        // K(j+3) and V buffer (r+1)%2 with V(j+1); one barrier per step, at its
        // end. Unrolled by six (3 K buffers, 2 V buffers, 2 score sets).
        for (int r = 0; r < nt; r += 6) {
            step(j_begin + r, sa0, sa1, sb0, sb1, Ks1, Ks0, Vs0, Vs1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
            if (r + 1 < nt) step(j_begin + r + 1, sb0, sb1, sa0, sa1, Ks2, Ks1, Vs1, Vs0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
            if (r + 2 < nt) step(j_begin + r + 2, sa0, sa1, sb0, sb1, Ks0, Ks2, Vs0, Vs1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
            if (r + 3 < nt) step(j_begin + r + 3, sb0, sb1, sa0, sa1, Ks1, Ks0, Vs1, Vs0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
            if (r + 4 < nt) step(j_begin + r + 4, sa0, sa1, sb0, sb1, Ks2, Ks1, Vs0, Vs1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
            if (r + 5 < nt) step(j_begin + r + 5, sb0, sb1, sa0, sa1, Ks0, Ks2, Vs1, Vs0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
        }
    }
    wait_vmcnt<0>();  // nothing is left in flight when the wave ends

    // Epilogue: O * (1/l), with the sink folded in first; rows that saw no
    // key are written as zeros. The log-sum-exp (natural log) goes to lse.
    float l_tot = sum_with_other_half(l_i);
    float m_fin = m_i;
    const float sink = p.sinks ? p.sinks[h] : -__builtin_inff();
    const bool nan_row = sink_gives_nan(sink);
    const float osc = p.sinks ? fold_sink(sink * kLog2e, m_fin, l_tot) : 1.f;
    const float inv = l_tot > 0.f ? (KV8 ? osc * p.v_scale : osc) / l_tot : 0.f;
    if (p.lse && hf == 0 && wave_live && my_q < sq)
        pf_store_lse(&p.lse[(lse_at + my_q) * p.n_q_heads + h], m_fin, l_tot, nan_row);
    pf_store_o16<BF16, NDT>(o, inv, (uint16_t*)p.o + o_at + (int64_t)min(my_q, sq - 1) * p.os.seq + (int64_t)h * p.os.head,
                            hf, nan_row, wave_live && my_q < sq);
}

// ---------------------------------------------------------------------------- D = 256, paired waves
// The pair's probability exchange: this lane's eight packed pairs into
// Xp[pair][half][0][lane] and Xp[pair][half][1][lane], 1 KB apart. The two
// LDS writes are issued from inline assembly: written in C++, the compiler
// guards the second one against the direct-to-LDS loads in flight (it does not
// tell them apart from the K/V tiles being filled) with a wait for every
// outstanding load, which drains the prefetch once per step. Only the barrier
// that follows orders them: barrier_lds waits for lgkmcnt(0), and its
// compiler fences keep every read of the exchange area on its far side.
__device__ __forceinline__ void xp_write(uint4* dst, const uint32_t (&pk)[8]) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)dst;
    const u32x4_t d0 = {pk[0], pk[1], pk[2], pk[3]}, d1 = {pk[4], pk[5], pk[6], pk[7]};
    asm volatile("ds_write_b128 %0, %1\n\tds_write_b128 %0, %2 offset:1024" ::"v"(a), "v"(d0), "v"(d1));
}

// prefill_pair: head_dim 256 at two waves per SIMD. A 32-row wave holding all
// of Q and O for 256 dims needs about 460 registers, which leaves one wave per
// SIMD and every stall exposed. Here the two waves of a pair share 32 query
// rows and split the work of each 64-key tile: wave half h computes the scores
// of keys 32h .. 32h+31 over all 256 dims (Q resident in full) and the output
// for dims 128h .. 128h+127 (that half of O resident). The pair exchanges its
// rows' tile maxima and its probabilities through LDS, so both waves run the
// same online softmax (the same m, the same rescale decisions, the same row
// sums over all 64 keys, in prefill_mfma's order) and each multiplies the
// tile's 64 probabilities into its half of V. Each wave needs about 230
// registers: eight waves (four pairs, 128 rows) per workgroup, two per SIMD.
// The arithmetic per row is prefill_mfma's, step for step, so the results are
// the same bits.
template <bool BF16, int MASK>
__global__ __launch_bounds__(512, 1) void prefill_pair(PrefillParams p) {
    constexpr int D = 256;
    constexpr int NW = 8;
    constexpr int PF_BM = 128;              // four pairs of 32 rows
    constexpr int PF_THREADS = 64 * NW;
    constexpr int CPR = D / 8;              // 16-byte chunks per row
    constexpr int TILE = PF_BN * D;
    constexpr int LPW = TILE / 512 / NW;    // 1 KB direct loads per wave per tile
    constexpr int NS = D / 16;              // k-steps of the score MFMAs
    constexpr int NDH = 4;                  // 32-wide d tiles in a wave's half of O^T
    constexpr int NPV = 4 * NDH;            // P V MFMAs per tile
    constexpr int VPRE = 4;                 // P V MFMAs whose fragments are in flight
    static_assert(LPW == 4 && NS % LPW == 0 && NPV % LPW == 0, "four direct loads per wave and tile");
    __shared__ __attribute__((aligned(16))) uint16_t Ks0[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Ks1[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vs0[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vs1[TILE];
    // Exchange between the waves of a pair: probabilities [pair][half][two
    // 16-byte chunks][lane] (a lane's 8 packed pairs), row maxima [pair][half][row].
    __shared__ __attribute__((aligned(16))) uint4 Xp[4][2][2][64];
    __shared__ float Xm[4][2][32];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pr = w & 3;       // pair: rows 32 pr .. 32 pr + 31 of the tile
    const int hh = w >> 2;      // half: keys 32 hh .. of each tile, dims 128 hh .. of O
    const int l32 = lane & 31;
    const int hf = lane >> 5;
    const int g = lane >> 4;
    const int r16 = lane & 15;

    // Workgroup -> (q tile, batch, q-head) as in prefill_mfma.
    const int nbh = p.batch * p.n_q_heads;
    int wid = (int)blockIdx.x;
    if (p.xcd_chunks) {
        const int G = p.group, round = 8 * G;
        const int full = ((int)gridDim.x / round) * round;
        if (wid < full) {
            const int xcd = wid & 7, k = wid >> 3;
            wid = ((k / G) * 8 + xcd) * G + k % G;
        }
    }
    const int qt = p.n_q_tiles - 1 - wid / nbh;
    const int bh = wid % nbh;
    const int b = bh / p.n_q_heads;
    const int h = bh % p.n_q_heads;
    const int hk = h / p.group;

    int sq = p.seqlen_q, skv = p.seqlen_kv;
    int64_t q_at = (int64_t)b * p.qs.batch, k_at = (int64_t)b * p.ks.batch, v_at = (int64_t)b * p.vs.batch,
            o_at = (int64_t)b * p.os.batch, lse_at = (int64_t)b * p.seqlen_q;
    if (p.cu_seqlens_q) {
        const int qs0 = p.cu_seqlens_q[b], ks0 = p.cu_seqlens_kv[b];
        sq = min(p.cu_seqlens_q[b + 1] - qs0, p.seqlen_q);
        skv = p.cu_seqlens_kv[b + 1] - ks0;
        q_at = (int64_t)qs0 * p.qs.seq;
        o_at = (int64_t)qs0 * p.os.seq;
        lse_at = qs0;
        k_at = (int64_t)ks0 * p.ks.seq;
        v_at = (int64_t)ks0 * p.vs.seq;
    }
    const int off = skv - sq;
    const int q0 = qt * PF_BM;
    if (q0 >= sq) return;  // a tile past this sequence's end (packed sequences only; uniform)
    const int qlast = min(q0 + PF_BM, sq) - 1;
    auto pos_of = [&](int i) -> int { return p.positions ? p.positions[lse_at + min(i, sq - 1)] : i + off; };
    int kv_lo = 0, kv_hi = skv;
    if (MASK >= kMaskCausal) kv_hi = min(kv_hi, pos_of(qlast) + 1);
    if (MASK == kMaskCausalWindow) kv_lo = max(0, pos_of(q0) - p.window + 1);
    const int j_begin = kv_lo / PF_BN;
    const int j_end = kv_hi > kv_lo ? (kv_hi + PF_BN - 1) / PF_BN : j_begin;

    const int wq0 = q0 + 32 * pr;
    const int wq1 = min(wq0 + 31, sq - 1);
    const bool wave_live = wq0 < sq;
    const int my_q = wq0 + l32;
    const int my_pos = pos_of(my_q);
    const int wpos0 = pos_of(wq0), wpos1 = pos_of(wq1);

    // Q (loaded in the prologue, after the first K/V tiles have been requested)
    s16x8 qf[NS];
    const uint16_t* qrow = (const uint16_t*)p.q + q_at + (int64_t)min(my_q, sq - 1) * p.qs.seq +
                           (int64_t)h * p.qs.head + 8 * hf;

    const uint16_t* kbase = (const uint16_t*)p.k + k_at + (int64_t)hk * p.ks.head;
    const uint16_t* vbase = (const uint16_t*)p.v + v_at + (int64_t)hk * p.vs.head;
    // K/V tiles: the direct-to-LDS staging of prefill_mfma (eight waves load a
    // tile together; rows outside [kv_lo, seqlen_kv) are clamped copies).
    const int key_min = kv_lo, key_max = skv - 1;
    constexpr int RPL = 64 / CPR;
    const int lrow = lane / CPR, lcs = lane % CPR;
    const uint32_t kx = 16u * (uint32_t)(lcs ^ lrow);
    const uint32_t vx = 16u * (uint32_t)(lcs ^ (4 * lrow));
    const uint32_t kl = 2u * (uint32_t)lrow * (uint32_t)p.ks.seq, vl = 2u * (uint32_t)lrow * (uint32_t)p.vs.seq;
    auto load_tile_impl = [&](uint16_t* dst, const uint16_t* base, int64_t seq, int j, uint32_t lane_row_off,
                              uint32_t lane_chunk_off, bool is_k) __attribute__((always_inline)) {
        const int kv0 = j * PF_BN;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)kv0 * seq), (short)0, 0x7fffffff, 0x00020000);
        if (kv0 >= key_min && kv0 + PF_BN - 1 <= key_max) {
#pragma unroll
            for (int ii = 0; ii < LPW; ++ii) {
                const int i = w * LPW + ii;
                const uint32_t u = is_k ? (2 * i) & 15 : 4 * ((2 * i) & 3);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 512 * i), 16,
                                                         lane_row_off + (lane_chunk_off ^ (16u * u)),
                                                         (uint32_t)(2 * RPL * i) * (uint32_t)seq, 0, 0);
            }
        } else {
            int lr = lrow;
            asm volatile("" : "+v"(lr));
#pragma unroll
            for (int ii = 0; ii < LPW; ++ii) {
                const int i = w * LPW + ii;
                const int row = RPL * i + lr, cs = lcs;
                const int key = min(max(kv0 + row, key_min), key_max);
                const int c = cs ^ (is_k ? pf_kswz<D>(row) : pf_vswz<D>(row));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 512 * i), 16,
                                                         2u * ((uint32_t)(key - kv0) * (uint32_t)seq + 8u * c), 0, 0, 0);
            }
        }
    };
    auto load_k_tile = [&](uint16_t* dst, int j) __attribute__((always_inline)) { load_tile_impl(dst, kbase, p.ks.seq, j, kl, kx, true); };
    auto load_v_tile = [&](uint16_t* dst, int j) __attribute__((always_inline)) { load_tile_impl(dst, vbase, p.vs.seq, j, vl, vx, false); };
    uint32_t kvo[LPW], vvo[LPW];
#pragma unroll
    for (int ii = 0; ii < LPW; ++ii) {
        const int i = w * LPW + ii;
        const uint32_t uk = (2 * i) & 15;
        const uint32_t uv = 4 * ((2 * i) & 3);
        uint32_t ko = kl + (kx ^ (16u * uk)) + (uint32_t)(2 * RPL * i) * (uint32_t)p.ks.seq;
        uint32_t vo = vl + (vx ^ (16u * uv)) + (uint32_t)(2 * RPL * i) * (uint32_t)p.vs.seq;
        asm volatile("" : "+v"(ko), "+v"(vo));
        kvo[ii] = ko;
        vvo[ii] = vo;
    }
    auto tile_rsrc = [&](const uint16_t* base, int64_t seq, int j) __attribute__((always_inline)) {
        const int kv0 = j * PF_BN;
        const uint32_t nrec =
            kv0 + PF_BN - 1 <= key_max ? 0x7fffffffu : 2u * ((uint32_t)(key_max - kv0) * (uint32_t)seq + (uint32_t)D);
        return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)kv0 * seq), (short)0, nrec, 0x00020000);
    };
    auto load_part = [&](uint16_t* dst, __amdgpu_buffer_rsrc_t rs, uint32_t voff, int ii) __attribute__((always_inline)) {
        const int i = w * LPW + ii;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 512 * i), 16, voff, 0, 0, 0);
    };

    constexpr float kLazyRescale = 8.0f;
    float m_i = kMaxInit, l_i = 0.f;
    f32x16 o[NDH];
#pragma unroll
    for (int dt = 0; dt < NDH; ++dt) o[dt] = f32x16{};
    const uint32_t one2 = BF16 ? 0x3F803F80u : 0x3C003C00u;

    auto tile_full = [&](int j) __attribute__((always_inline)) {
        const int kv0 = j * PF_BN;
        bool f = kv0 + PF_BN <= skv;
        if (MASK >= kMaskCausal) f &= kv0 + PF_BN - 1 <= wpos0;
        if (MASK == kMaskCausalWindow) f &= kv0 >= wpos1 - p.window + 1;
        return f;
    };
    // Fragment offsets: this wave's 32-key block of K starts 32 rows into the
    // tile; its half of V^T is d tiles 4 hh .. 4 hh + 3 (chunk XOR 16 hh).
    const uint32_t kfrag = ((uint32_t)(l32 * D * 2) | (16u * (uint32_t)(hf ^ pf_kswz<D>(l32)))) + (uint32_t)hh * (32u * D * 2);
    const int vr0 = 4 * hf + (r16 >> 2);
    const int vcl = 2 * (g & 1) + ((r16 & 3) >> 1);
    const uint32_t vfrag = ((uint32_t)(vr0 * D * 2) | (16u * (uint32_t)(vcl ^ pf_vswz<D>(vr0))) | (8u * (r16 & 1))) ^
                           (256u * (uint32_t)hh);
    auto opaque = [](uint32_t x) __attribute__((always_inline)) {
        asm volatile("" : "+v"(x));
        return x;
    };
    auto lds_frag8 = [](const uint16_t* base, uint32_t byte_off) __attribute__((always_inline)) {
        return *(const s16x8*)((const char*)base + byte_off);
    };
    int key_hi = skv - 1, key_lo = 0;
    if (MASK >= kMaskCausal) key_hi = min(key_hi, my_pos);
    if (MASK == kMaskCausalWindow) key_lo = max(key_lo, my_pos - p.window + 1);
    const bool none_visible = key_hi < key_lo;
    const uint32_t key_span = none_visible ? 0u : (uint32_t)(key_hi - key_lo);
    if (none_visible) key_lo = INT_MIN / 2;
    // this wave's block of a tile: keys kv0 + 32 hh + 8 (r / 4) + 4 hf + r % 4 in register r
    auto mask_block = [&](f32x16& sacc, int kv0) __attribute__((always_inline)) {
        const int base = kv0 + 32 * hh + 4 * hf - key_lo;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const uint32_t d = (uint32_t)(base + 8 * (r >> 2) + (r & 3));
            sacc[r] = d <= key_span ? sacc[r] : kMaskedScore;
        }
    };
    auto max_block = [&](const f32x16& s) __attribute__((always_inline)) {
        float mx = kMaskedScore;
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = max3f(mx, s[r], s[r + 1]);
        return max_with_other_half(mx);
    };
    auto rescale = [&](float mx) __attribute__((always_inline)) {
        const float m_cand = mx * p.c;
        const bool grow = m_cand > m_i + kLazyRescale;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = grow ? m_cand : m_i;
            const float alpha = fast_exp2(m_i - m_new);
            m_i = m_new;
            l_i *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDH; ++dt) o[dt] *= alpha;
        }
    };
    // The pair's tile max: this wave's (masked) block max against its partner's.
    auto exchange_max = [&](float mx) __attribute__((always_inline)) {
        if (hf == 0) Xm[pr][hh][l32] = mx;
        return mx;
    };

    // Step j (as prefill_mfma's): the score MFMAs of tile j+1 (this wave's
    // block) beside the exponentials of tile j; this wave's probabilities go to
    // LDS; a barrier (which also publishes V(j)); both halves' probabilities
    // are read back in order; the P V MFMAs of tile j into this wave's half of
    // O beside the raw row max of tile j+1; the row sums of all 64
    // probabilities; the tile max of j+1 goes to LDS; a barrier (K(j+2) in);
    // the partner's max settles m for tile j+1. Loads: V(j+1) in the first
    // part, K(j+3) in the second, as in prefill_mfma.
    const int j_last = j_end - 1;
    auto step = [&](int j, f32x16& c, f32x16& n, uint16_t* Kn, uint16_t* Vc, uint16_t* Vl) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t vrs = tile_rsrc(vbase, p.vs.seq, min(j + 1, j_last));
        const uint32_t kf = opaque(kfrag);
        const uint32_t vf = opaque(vfrag);
        s16x8 ka[NS];
        s16x8 vb[NPV];
        uint32_t pk[8];
        auto kread = [&](int s) __attribute__((always_inline)) { ka[s] = lds_frag8(Kn, kf ^ (32u * s)); };
        auto vread = [&](int i) __attribute__((always_inline)) {
            const int u = i / NDH, dt = i % NDH;
            const char* vb0 = (const char*)Vc + (vf ^ (64u * dt));
            vb[i] = concat4(lds_read_tr16((const uint16_t*)(vb0 + 2 * D * (16 * u))),
                            lds_read_tr16((const uint16_t*)(vb0 + 2 * D * (16 * u + 8))));
        };
        const float neg_m = -m_i;
        auto prob_pair = [&](int i) __attribute__((always_inline)) {
            pk[i] = pack2_16<BF16>(fast_exp2(fmaf(c[2 * i], p.c, neg_m)), fast_exp2(fmaf(c[2 * i + 1], p.c, neg_m)));
            asm volatile("" ::"v"(pk[i]));
        };
        kread(0);
        kread(1);
        sched_fence();
        n = f32x16{};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            n = mfma32x32x16<BF16>(ka[s], qf[s], n);
            if (s % (NS / LPW) == 0) load_part(Vl, vrs, vvo[s / (NS / LPW)], s / (NS / LPW));
            if (s + 2 < NS) kread(s + 2);
            if (s % 2 == 1) prob_pair(s / 2);
            sched_fence();
        }
        xp_write(&Xp[pr][hh][0][lane], pk);
        // V(j) in; both halves' P(j) written; every wave is past its reads of K(j+1).
        wait_vmcnt<2 * LPW>();
        barrier_lds();
        const __amdgpu_buffer_rsrc_t krs = tile_rsrc(kbase, p.ks.seq, min(j + 3, j_last));
        uint4 pq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pq[e] = Xp[pr][e >> 1][e & 1][lane];
#pragma unroll
        for (int i = 0; i < VPRE; ++i) vread(i);
        sched_fence();
        float mx = kMaskedScore;
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            const int u = i / NDH, dt = i % NDH;
            o[dt] = mfma32x32x16<BF16>(vb[i], __builtin_bit_cast(s16x8, pq[u]), o[dt]);
            if (i % (NPV / LPW) == 0) load_part(Kn, krs, kvo[i / (NPV / LPW)], i / (NPV / LPW));
            if (i + VPRE < NPV) vread(i + VPRE);
            if (i % 2 == 0) mx = max3f(mx, n[i], n[i + 1]);
            sched_fence();
        }
        // row sums of the tile's 64 probabilities, in prefill_mfma's order
        const uint32_t* pw = (const uint32_t*)pq;
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            ps0 = dot2_16<BF16>(pw[e], one2, ps0);
            ps1 = dot2_16<BF16>(pw[e + 1], one2, ps1);
        }
        l_i += ps0 + ps1;
        mx = max_with_other_half(mx);
        if (!(wave_live && tile_full(j + 1))) {
            mask_block(n, (j + 1) * PF_BN);
            mx = fminf(mx, max_block(n));
        }
        exchange_max(mx);
        // K(j+2) in; both halves' tile maxima written; every wave is past its reads of V(j).
        wait_vmcnt<2 * LPW>();
        barrier_lds();
        rescale(fmaxf(mx, Xm[pr][hh ^ 1][l32]));
    };

    f32x16 sa, sb;
    const int nt = j_end - j_begin;
    if (nt > 0) {
        // The first refill of Vs1 may be range-limited: start it from zeros.
#pragma unroll
        for (int c = tid; c < TILE / 8; c += PF_THREADS) *(uint4*)(Vs1 + 8 * c) = make_uint4(0, 0, 0, 0);
        // K(j_begin) and Q first: the first scores wait for those only, while
        // V(j_begin) and K(j_begin + 1) arrive behind them.
        load_k_tile(Ks0, j_begin);
        pf_load_q<D>(qf, qrow, my_q < sq, p.qflip);
        load_v_tile(Vs0, j_begin);
        load_k_tile(Ks1, min(j_begin + 1, j_last));
        wait_vmcnt<2 * LPW>();
        barrier_lds();
        {
            const uint32_t kf = opaque(kfrag);
            sa = f32x16{};
#pragma unroll
            for (int s = 0; s < NS; ++s) sa = mfma32x32x16<BF16>(lds_frag8(Ks0, kf ^ (32u * s)), qf[s], sa);
        }
        if (!(wave_live && tile_full(j_begin))) mask_block(sa, j_begin * PF_BN);
        const float mx = exchange_max(max_block(sa));
        // V(j_begin) and K(j_begin + 1) in; the tile maxima are written; every wave is past its reads of K(j_begin)
        wait_vmcnt<0>();
        barrier_lds();
        rescale(fmaxf(mx, Xm[pr][hh ^ 1][l32]));
        load_k_tile(Ks0, min(j_begin + 2, j_last));
    }
    for (int r = 0; r < nt; r += 2) {
        step(j_begin + r, sa, sb, Ks1, Vs0, Vs1);
        if (r + 1 < nt) step(j_begin + r + 1, sb, sa, Ks0, Vs1, Vs0);
    }
    wait_vmcnt<0>();

    float l_tot = sum_with_other_half(l_i);
    float m_fin = m_i;
    const float sink = p.sinks ? p.sinks[h] : -__builtin_inff();
    const bool nan_row = sink_gives_nan(sink);
    const float osc = p.sinks ? fold_sink(sink * kLog2e, m_fin, l_tot) : 1.f;
    const float inv = l_tot > 0.f ? osc / l_tot : 0.f;
    if (p.lse && hh == 0 && hf == 0 && wave_live && my_q < sq)
        pf_store_lse(&p.lse[(lse_at + my_q) * p.n_q_heads + h], m_fin, l_tot, nan_row);
    pf_store_o16<BF16, NDH>(o, inv,
                            (uint16_t*)p.o + o_at + (int64_t)min(my_q, sq - 1) * p.os.seq + (int64_t)h * p.os.head + 128 * hh,
                            hf, nan_row, wave_live && my_q < sq);
}

// ---------------------------------------------------------------------------- D = 256, paired waves, persistent
// prefill_pair_items: prefill_pair as a persistent loop over q tiles, for the
// launches whose q tiles all carry the same kind of work (a sliding window or
// no mask over one fixed-size sequence per batch entry). A workgroup that ends
// pays for its successor's first loads (Q and three K/V tiles, about 224 KB
// per CU) before the successor's first MFMA, and for its own stores; measured
// on the D = 256 window workload that is about a quarter of each workgroup's
// time. Here one workgroup per CU takes the items (q tile, batch, q-head)
// blockIdx.x, blockIdx.x + gridDim.x, ... and the key loop runs on from one
// item into the next: the tile stream (V one tile ahead, K three ahead)
// continues into the next item's first tiles, the next item's Q is loaded
// right after the score MFMAs that last use the current Q (one step before
// it is needed), and the finished item's O is stored while the next one
// starts. Every item covers an even number of key tiles (host-checked), so
// every item starts on the same buffer parity and the step sequence of an
// item is: pairs of ordinary steps, then a step that loads the next Q, then
// the step that ends the item. The host also requires seqlen_kv and the
// call's first visible key to be multiples of 64, so every tile loaded lies
// whole inside [first visible key, seqlen_kv) and no load needs clamping
// (tile rows below an item's own first key are keys that earlier q tiles
// see, masked for this item's rows). The arithmetic per row is prefill_pair's.
constexpr int kStepPlain = 0, kStepNextQ = 1, kStepLast = 2;

template <bool BF16, int MASK>
__global__ __launch_bounds__(512, 1) void prefill_pair_items(PrefillParams p) {
    static_assert(MASK != kMaskCausal, "causal q tiles differ in work: prefill_pair");
    constexpr int D = 256;
    constexpr int NW = 8;
    constexpr int PF_BM = 128;
    constexpr int PF_THREADS = 64 * NW;
    constexpr int CPR = D / 8;
    constexpr int TILE = PF_BN * D;
    constexpr int LPW = TILE / 512 / NW;
    constexpr int NS = D / 16;
    constexpr int NDH = 4;
    constexpr int NPV = 4 * NDH;
    constexpr int VPRE = 4;
    static_assert(LPW == 4 && NS % LPW == 0 && NPV % LPW == 0, "four direct loads per wave and tile");
    __shared__ __attribute__((aligned(16))) uint16_t Ks0[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Ks1[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vs0[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vs1[TILE];
    __shared__ __attribute__((aligned(16))) uint4 Xp[4][2][2][64];
    __shared__ float Xm[4][2][32];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pr = w & 3;
    const int hh = w >> 2;
    const int l32 = lane & 31;
    const int hf = lane >> 5;
    const int g = lane >> 4;
    const int r16 = lane & 15;

    const int nbh = p.batch * p.n_q_heads;
    const int total = p.n_q_tiles * nbh;
    const int sq = p.seqlen_q, skv = p.seqlen_kv, off = skv - sq;
    const int key_max = skv - 1;
    const int P = (int)gridDim.x;
    const int M = (total - (int)blockIdx.x + P - 1) / P;  // this workgroup's items (>= 1: the grid is <= total)

    // Item m of this workgroup -> (q tile, batch, q-head) and its key tiles,
    // in prefill_pair's logical order (XCD chunks included).
    struct Item {
        int b, h, hk, q0, jb, nt;
    };
    auto item = [&](int m) __attribute__((always_inline)) {
        int wid = (int)blockIdx.x + m * P;
        if (p.xcd_chunks) {
            const int G = p.group, round = 8 * G;
            const int full = (total / round) * round;
            if (wid < full) {
                const int xcd = wid & 7, k = wid >> 3;
                wid = ((k / G) * 8 + xcd) * G + k % G;
            }
        }
        Item it;
        const int qt = p.n_q_tiles - 1 - wid / nbh;
        const int bh = wid % nbh;
        it.b = bh / p.n_q_heads;
        it.h = bh % p.n_q_heads;
        it.hk = it.h / p.group;
        it.q0 = qt * PF_BM;
        const int qlast = min(it.q0 + PF_BM, sq) - 1;
        int kv_lo = 0, kv_hi = skv;
        if (MASK >= kMaskCausal) kv_hi = min(kv_hi, qlast + off + 1);
        if (MASK == kMaskCausalWindow) kv_lo = max(0, it.q0 + off - p.window + 1);
        it.jb = kv_lo / PF_BN;
        it.nt = (kv_hi + PF_BN - 1) / PF_BN - it.jb;  // even and >= 2 (host-checked)
        return it;
    };
    // This lane's row of an item: validity, positions, visible key range.
    struct Rows {
        int my_q, wpos0, wpos1, key_lo;
        uint32_t key_span;
        bool live;
    };
    auto rows_of = [&](const Item& it) __attribute__((always_inline)) {
        Rows R;
        const int wq0 = it.q0 + 32 * pr;
        const int wq1 = min(wq0 + 31, sq - 1);
        R.live = wq0 < sq;
        R.my_q = wq0 + l32;
        const int my_pos = R.my_q + off;
        R.wpos0 = wq0 + off;
        R.wpos1 = wq1 + off;
        int key_hi = skv - 1, key_lo = 0;
        if (MASK >= kMaskCausal) key_hi = min(key_hi, my_pos);
        if (MASK == kMaskCausalWindow) key_lo = max(key_lo, my_pos - p.window + 1);
        const bool none_visible = key_hi < key_lo;
        R.key_span = none_visible ? 0u : (uint32_t)(key_hi - key_lo);
        R.key_lo = none_visible ? INT_MIN / 2 : key_lo;
        return R;
    };
    auto kbase_of = [&](const Item& it) __attribute__((always_inline)) {
        return (const uint16_t*)p.k + (int64_t)it.b * p.ks.batch + (int64_t)it.hk * p.ks.head;
    };
    auto vbase_of = [&](const Item& it) __attribute__((always_inline)) {
        return (const uint16_t*)p.v + (int64_t)it.b * p.vs.batch + (int64_t)it.hk * p.vs.head;
    };
    auto qrow_of = [&](const Item& it, const Rows& R) __attribute__((always_inline)) {
        return (const uint16_t*)p.q + (int64_t)it.b * p.qs.batch + (int64_t)min(R.my_q, sq - 1) * p.qs.seq +
               (int64_t)it.h * p.qs.head + 8 * hf;
    };

    // K/V staging as in prefill_pair, every tile whole (see above): one
    // descriptor per tile, lane offsets computed once.
    constexpr int RPL = 64 / CPR;
    const int lrow = lane / CPR, lcs = lane % CPR;
    const uint32_t kx = 16u * (uint32_t)(lcs ^ lrow);
    const uint32_t vx = 16u * (uint32_t)(lcs ^ (4 * lrow));
    const uint32_t kl = 2u * (uint32_t)lrow * (uint32_t)p.ks.seq, vl = 2u * (uint32_t)lrow * (uint32_t)p.vs.seq;
    uint32_t kvo[LPW], vvo[LPW];
#pragma unroll
    for (int ii = 0; ii < LPW; ++ii) {
        const int i = w * LPW + ii;
        const uint32_t uk = (2 * i) & 15;
        const uint32_t uv = 4 * ((2 * i) & 3);
        uint32_t ko = kl + (kx ^ (16u * uk)) + (uint32_t)(2 * RPL * i) * (uint32_t)p.ks.seq;
        uint32_t vo = vl + (vx ^ (16u * uv)) + (uint32_t)(2 * RPL * i) * (uint32_t)p.vs.seq;
        asm volatile("" : "+v"(ko), "+v"(vo));
        kvo[ii] = ko;
        vvo[ii] = vo;
    }
    auto k_rsrc = [&](const Item& it, int j) __attribute__((always_inline)) {
        return __builtin_amdgcn_make_buffer_rsrc((void*)(kbase_of(it) + (int64_t)j * PF_BN * p.ks.seq), (short)0,
                                                 0x7fffffff, 0x00020000);
    };
    auto v_rsrc = [&](const Item& it, int j) __attribute__((always_inline)) {
        return __builtin_amdgcn_make_buffer_rsrc((void*)(vbase_of(it) + (int64_t)j * PF_BN * p.vs.seq), (short)0,
                                                 0x7fffffff, 0x00020000);
    };
    auto load_part = [&](uint16_t* dst, __amdgpu_buffer_rsrc_t rs, uint32_t voff, int ii) __attribute__((always_inline)) {
        const int i = w * LPW + ii;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 512 * i), 16, voff, 0, 0, 0);
    };
    auto load_k_tile = [&](uint16_t* dst, const Item& it, int j) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs = k_rsrc(it, j);
#pragma unroll
        for (int ii = 0; ii < LPW; ++ii) load_part(dst, rs, kvo[ii], ii);
    };
    auto load_v_tile = [&](uint16_t* dst, const Item& it, int j) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs = v_rsrc(it, j);
#pragma unroll
        for (int ii = 0; ii < LPW; ++ii) load_part(dst, rs, vvo[ii], ii);
    };

    constexpr float kLazyRescale = 8.0f;
    float m_i = kMaxInit, l_i = 0.f;
    f32x16 o[NDH];
#pragma unroll
    for (int dt = 0; dt < NDH; ++dt) o[dt] = f32x16{};
    const uint32_t one2 = BF16 ? 0x3F803F80u : 0x3C003C00u;

    auto tile_full = [&](int j, const Rows& R) __attribute__((always_inline)) {
        const int kv0 = j * PF_BN;
        bool f = kv0 + PF_BN <= skv;
        if (MASK >= kMaskCausal) f &= kv0 + PF_BN - 1 <= R.wpos0;
        if (MASK == kMaskCausalWindow) f &= kv0 >= R.wpos1 - p.window + 1;
        return f;
    };
    const uint32_t kfrag = ((uint32_t)(l32 * D * 2) | (16u * (uint32_t)(hf ^ pf_kswz<D>(l32)))) + (uint32_t)hh * (32u * D * 2);
    const int vr0 = 4 * hf + (r16 >> 2);
    const int vcl = 2 * (g & 1) + ((r16 & 3) >> 1);
    const uint32_t vfrag = ((uint32_t)(vr0 * D * 2) | (16u * (uint32_t)(vcl ^ pf_vswz<D>(vr0))) | (8u * (r16 & 1))) ^
                           (256u * (uint32_t)hh);
    auto opaque = [](uint32_t x) __attribute__((always_inline)) {
        asm volatile("" : "+v"(x));
        return x;
    };
    auto lds_frag8 = [](const uint16_t* base, uint32_t byte_off) __attribute__((always_inline)) {
        return *(const s16x8*)((const char*)base + byte_off);
    };
    auto mask_block = [&](f32x16& sacc, int kv0, const Rows& R) __attribute__((always_inline)) {
        const int base = kv0 + 32 * hh + 4 * hf - R.key_lo;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const uint32_t d = (uint32_t)(base + 8 * (r >> 2) + (r & 3));
            sacc[r] = d <= R.key_span ? sacc[r] : kMaskedScore;
        }
    };
    auto max_block = [&](const f32x16& sc) __attribute__((always_inline)) {
        float mx = kMaskedScore;
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = max3f(mx, sc[r], sc[r + 1]);
        return max_with_other_half(mx);
    };
    auto rescale = [&](float mx) __attribute__((always_inline)) {
        const float m_cand = mx * p.c;
        const bool grow = m_cand > m_i + kLazyRescale;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = grow ? m_cand : m_i;
            const float alpha = fast_exp2(m_i - m_new);
            m_i = m_new;
            l_i *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDH; ++dt) o[dt] *= alpha;
        }
    };
    auto exchange_max = [&](float mx) __attribute__((always_inline)) {
        if (hf == 0) Xm[pr][hh][l32] = mx;
        return mx;
    };
    // The finished item's output (and log-sum-exp), then a fresh softmax state.
    auto finish = [&](const Item& it, const Rows& R) __attribute__((always_inline)) {
        float l_tot = sum_with_other_half(l_i);
        float m_fin = m_i;
        const float sink = p.sinks ? p.sinks[it.h] : -__builtin_inff();
        const bool nan_row = sink_gives_nan(sink);
        const float osc = p.sinks ? fold_sink(sink * kLog2e, m_fin, l_tot) : 1.f;
        const float inv = l_tot > 0.f ? osc / l_tot : 0.f;
        if (p.lse && hh == 0 && hf == 0 && R.live && R.my_q < sq)
            pf_store_lse(&p.lse[((int64_t)it.b * sq + R.my_q) * p.n_q_heads + it.h], m_fin, l_tot, nan_row);
        pf_store_o16<BF16, NDH>(o, inv,
                                (uint16_t*)p.o + (int64_t)it.b * p.os.batch + (int64_t)min(R.my_q, sq - 1) * p.os.seq +
                                    (int64_t)it.h * p.os.head + 128 * hh,
                                hf, nan_row, R.live && R.my_q < sq);
#pragma unroll
        for (int dt = 0; dt < NDH; ++dt) o[dt] = f32x16{};
        l_i = 0.f;
        m_i = kMaxInit;
    };

    s16x8 qf[NS];
    Item cur = item(0);
    Rows cr = rows_of(cur);
    Item nx = M > 1 ? item(1) : cur;  // the current item stands in for a missing next one
    Rows nr = rows_of(nx);
    int m_cur = 0;

    // Step r of item cur (prefill_pair's step): the score MFMAs of the tile
    // after r (the next item's first tile in the last step, with the next Q
    // and masked for the next item's rows) beside the exponentials of tile r;
    // P exchange; P V of tile r; row sums; the tile max of the tile after r;
    // then, in the last step, the item's output and a fresh state before m
    // is settled for the next item. Loads: V one tile ahead and K three
    // ahead in the stream of tiles (cur's, then nx's, then the item after
    // nx when nx has two tiles); the step before the last also loads the
    // next item's Q, and its waits allow for those NS loads.
    auto step = [&](int kind, int r, f32x16& c, f32x16& n, uint16_t* Kn, uint16_t* Vc, uint16_t* Vl)
                    __attribute__((always_inline)) {
        const int j = cur.jb + r;
        const uint32_t kf = opaque(kfrag);
        const uint32_t vf = opaque(vfrag);
        s16x8 ka[NS];
        s16x8 vb[NPV];
        uint32_t pk[8];
        auto kread = [&](int s) __attribute__((always_inline)) { ka[s] = lds_frag8(Kn, kf ^ (32u * s)); };
        auto vread = [&](int i) __attribute__((always_inline)) {
            const int u = i / NDH, dt = i % NDH;
            const char* vb0 = (const char*)Vc + (vf ^ (64u * dt));
            vb[i] = concat4(lds_read_tr16((const uint16_t*)(vb0 + 2 * D * (16 * u))),
                            lds_read_tr16((const uint16_t*)(vb0 + 2 * D * (16 * u + 8))));
        };
        const float neg_m = -m_i;
        auto prob_pair = [&](int i) __attribute__((always_inline)) {
            pk[i] = pack2_16<BF16>(fast_exp2(fmaf(c[2 * i], p.c, neg_m)), fast_exp2(fmaf(c[2 * i + 1], p.c, neg_m)));
            asm volatile("" ::"v"(pk[i]));
        };
        // the V tile one ahead and the K tile three ahead in the stream
        const __amdgpu_buffer_rsrc_t vrs = kind == kStepLast ? v_rsrc(nx, nx.jb) : v_rsrc(cur, j + 1);
        __amdgpu_buffer_rsrc_t krs;
        if (kind == kStepPlain) {
            krs = r + 3 < cur.nt ? k_rsrc(cur, j + 3) : k_rsrc(nx, nx.jb);
        } else if (kind == kStepNextQ) {
            krs = k_rsrc(nx, nx.jb + 1);
        } else if (nx.nt > 2) {
            krs = k_rsrc(nx, nx.jb + 2);
        } else {
            const Item n2 = m_cur + 2 < M ? item(m_cur + 2) : nx;
            krs = k_rsrc(n2, n2.jb);
        }
        kread(0);
        kread(1);
        sched_fence();
        n = f32x16{};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            n = mfma32x32x16<BF16>(ka[s], qf[s], n);
            if (s % (NS / LPW) == 0) load_part(Vl, vrs, vvo[s / (NS / LPW)], s / (NS / LPW));
            if (s + 2 < NS) kread(s + 2);
            if (s % 2 == 1) prob_pair(s / 2);
            sched_fence();
        }
        if (kind == kStepNextQ) pf_load_q<D>(qf, qrow_of(nx, nr), nr.my_q < sq, p.qflip);
        xp_write(&Xp[pr][hh][0][lane], pk);
        // V(j) in; both halves' P(j) written; every wave is past its reads of the K tile after j.
        if (kind == kStepNextQ) wait_vmcnt<2 * LPW + NS>(); else wait_vmcnt<2 * LPW>();
        barrier_lds();
        uint4 pq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pq[e] = Xp[pr][e >> 1][e & 1][lane];
#pragma unroll
        for (int i = 0; i < VPRE; ++i) vread(i);
        sched_fence();
        float mx = kMaskedScore;
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            const int u = i / NDH, dt = i % NDH;
            o[dt] = mfma32x32x16<BF16>(vb[i], __builtin_bit_cast(s16x8, pq[u]), o[dt]);
            if (i % (NPV / LPW) == 0) load_part(Kn, krs, kvo[i / (NPV / LPW)], i / (NPV / LPW));
            if (i + VPRE < NPV) vread(i + VPRE);
            if (i % 2 == 0) mx = max3f(mx, n[i], n[i + 1]);
            sched_fence();
        }
        const uint32_t* pw = (const uint32_t*)pq;
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            ps0 = dot2_16<BF16>(pw[e], one2, ps0);
            ps1 = dot2_16<BF16>(pw[e + 1], one2, ps1);
        }
        l_i += ps0 + ps1;
        mx = max_with_other_half(mx);
        const Rows& sr = kind == kStepLast ? nr : cr;
        const int sj = kind == kStepLast ? nx.jb : j + 1;
        if (!(sr.live && tile_full(sj, sr))) {
            mask_block(n, sj * PF_BN, sr);
            mx = fminf(mx, max_block(n));
        }
        exchange_max(mx);
        // The K tile two ahead is in; both halves' tile maxima written; every wave is past its reads of V(j).
        if (kind == kStepNextQ) wait_vmcnt<2 * LPW + NS>(); else wait_vmcnt<2 * LPW>();
        barrier_lds();
        if (kind == kStepLast) finish(cur, cr);
        rescale(fmaxf(mx, Xm[pr][hh ^ 1][l32]));
    };

    // Prologue (the first item): K(jb) and Q first, then V(jb) and K(jb+1);
    // the first scores and their m; then the K tile two ahead.
    f32x16 sa, sb;
#pragma unroll
    for (int c = tid; c < TILE / 8; c += PF_THREADS) *(uint4*)(Vs1 + 8 * c) = make_uint4(0, 0, 0, 0);
    {
        uint4 qraw[NS];
        load_k_tile(Ks0, cur, cur.jb);
        pf_load_q_raw<D>(qraw, qrow_of(cur, cr));
        sched_fence();
        load_v_tile(Vs0, cur, cur.jb);
        load_k_tile(Ks1, cur, cur.jb + 1);
        wait_vmcnt<2 * LPW>();
        barrier_lds();
        pf_mask_q<D>(qf, qraw, cr.my_q < sq, p.qflip);
    }
    {
        const uint32_t kf = opaque(kfrag);
        sa = f32x16{};
#pragma unroll
        for (int s = 0; s < NS; ++s) sa = mfma32x32x16<BF16>(lds_frag8(Ks0, kf ^ (32u * s)), qf[s], sa);
    }
    if (!(cr.live && tile_full(cur.jb, cr))) mask_block(sa, cur.jb * PF_BN, cr);
    {
        const float mx = exchange_max(max_block(sa));
        wait_vmcnt<0>();
        barrier_lds();
        rescale(fmaxf(mx, Xm[pr][hh ^ 1][l32]));
    }
    if (cur.nt > 2) load_k_tile(Ks0, cur, cur.jb + 2);
    else load_k_tile(Ks0, nx, nx.jb);

    for (int m = 0; m < M; ++m) {
        const int nt = cur.nt;
        for (int r = 0; r < nt - 2; r += 2) {
            step(kStepPlain, r, sa, sb, Ks1, Vs0, Vs1);
            step(kStepPlain, r + 1, sb, sa, Ks0, Vs1, Vs0);
        }
        step(kStepNextQ, nt - 2, sa, sb, Ks1, Vs0, Vs1);
        step(kStepLast, nt - 1, sb, sa, Ks0, Vs1, Vs0);
        cur = nx;
        cr = nr;
        m_cur = m + 1;
        nx = m + 2 < M ? item(m + 2) : cur;
        nr = rows_of(nx);
    }
    wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------- FP8 K/V
// prefill_f8kv: prefill for K and V stored as FP8 E4M3 codes with one scale
// per tensor (a code stands for scale times its value; the host folds K's
// scale into c and V's scale multiplies the output). The FP8 variant of the
// decode page's quantised cache, applied to the prefill's K/V stream. Each
// 64-key tile is read into registers (16 codes per load), widened exactly to
// the 16-bit type (gfx950's v_cvt_scalef32_pk_*_fp8 with scale 1) and written
// to LDS in prefill_mfma's swizzled tile layout, so the fragment reads, the
// masks, the online softmax with its lazy rescale and the epilogue are
// prefill_mfma's. Two LDS buffers per tensor: tile j+1 is requested before
// the MFMAs of tile j and written after them, with one barrier per tile.
// Four waves of 32 query rows; no software pipelining across tiles. (The wide
// D = 128 grids go to prefill_mfma with FP8 staging instead.)
template <bool BF16, int D, int MASK, int NW>
__global__ __launch_bounds__(64 * NW, (NW == 8 || D >= 256 ? 1 : 2)) void prefill_f8kv(PrefillParams p) {
    constexpr int PF_BM = PF_ROWS_PER_WAVE * NW;
    constexpr int TILE = PF_BN * D;
    constexpr int NDT = D / 32;
    constexpr int CH8 = D / 16;             // 16-byte chunks of codes per row
    constexpr int NT = 64 * NW;             // threads
    constexpr int NLD = PF_BN * CH8 / NT;   // chunks per thread per tile and tensor
    static_assert(NLD >= 1, "every thread loads part of each tile");
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hf = lane >> 5;
    const int g = lane >> 4;
    const int r16 = lane & 15;

    // Workgroup -> (q tile, batch, q-head), heaviest causal tiles first.
    const int nbh = p.batch * p.n_q_heads;
    const int wid = (int)blockIdx.x;
    const int qt = p.n_q_tiles - 1 - wid / nbh;
    const int bh = wid % nbh;
    const int b = bh / p.n_q_heads;
    const int h = bh % p.n_q_heads;
    const int hk = h / p.group;
    const int sq = p.seqlen_q, skv = p.seqlen_kv;
    const int off = skv - sq;  // query row i sits at position i + off
    const int q0 = qt * PF_BM;
    const int qlast = min(q0 + PF_BM, sq) - 1;
    int kv_lo = 0, kv_hi = skv;
    if (MASK >= kMaskCausal) kv_hi = min(kv_hi, qlast + off + 1);
    if (MASK == kMaskCausalWindow) kv_lo = max(0, q0 + off - p.window + 1);
    const int j_begin = kv_lo / PF_BN;
    const int j_end = kv_hi > kv_lo ? (kv_hi + PF_BN - 1) / PF_BN : j_begin;

    const int wq0 = q0 + 32 * w;
    const int wq1 = min(wq0 + 31, sq - 1);
    const bool wave_live = wq0 < sq;
    const int my_q = wq0 + l32;
    const int my_pos = my_q + off;
    const int wpos0 = wq0 + off, wpos1 = wq1 + off;

    // Q: loaded after the first K/V tile has been requested (the row is clamped
    // into the sequence; rows past it are zeroed)
    s16x8 qf[D / 16];
    const uint16_t* qrow = (const uint16_t*)p.q + (int64_t)b * p.qs.batch + (int64_t)min(my_q, sq - 1) * p.qs.seq +
                           (int64_t)h * p.qs.head + 8 * hf;

    // Tile staging. Thread chunk c = tid + NT i covers codes 16 (c % CH8) ..
    // +16 of tile row c / CH8; rows outside [kv_lo, skv) read the nearest valid
    // row (masked later), so every load stays inside the visible key range.
    const uint8_t* kb8 = (const uint8_t*)p.k + (int64_t)b * p.ks.batch + (int64_t)hk * p.ks.head;
    const uint8_t* vb8 = (const uint8_t*)p.v + (int64_t)b * p.vs.batch + (int64_t)hk * p.vs.head;
    const int key_min = kv_lo, key_max = skv - 1;
    uint4 kr[NLD], vr[NLD];
    auto fetch = [&](int j) __attribute__((always_inline)) {
        const int kv0 = j * PF_BN;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int c = tid + NT * i;
            const int key = min(max(kv0 + c / CH8, key_min), key_max);
            const int col = 16 * (c % CH8);
            kr[i] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)(kb8 + (int64_t)key * p.ks.seq + col)));
            vr[i] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)(vb8 + (int64_t)key * p.vs.seq + col)));
        }
    };
    auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int c = tid + NT * i;
            const int row = c / CH8, cc = c % CH8;
            uint4 lo, hi;
            char* krow = (char*)Ks[buf] + row * D * 2;
            widen_e4m3x16<BF16>(kr[i], lo, hi);
            *(uint4*)(krow + 16 * ((2 * cc) ^ pf_kswz<D>(row))) = lo;
            *(uint4*)(krow + 16 * ((2 * cc + 1) ^ pf_kswz<D>(row))) = hi;
            char* vrow = (char*)Vs[buf] + row * D * 2;
            widen_e4m3x16<BF16>(vr[i], lo, hi);
            *(uint4*)(vrow + 16 * ((2 * cc) ^ pf_vswz<D>(row))) = lo;
            *(uint4*)(vrow + 16 * ((2 * cc + 1) ^ pf_vswz<D>(row))) = hi;
        }
    };

    // Fragment offsets and per-tile steps as in prefill_mfma.
    const uint32_t kfrag = (uint32_t)(l32 * D * 2) | (16u * (uint32_t)(hf ^ pf_kswz<D>(l32)));
    const int vr0 = 4 * hf + (r16 >> 2);
    const int vcl = 2 * (g & 1) + ((r16 & 3) >> 1);
    const uint32_t vfrag = (uint32_t)(vr0 * D * 2) | (16u * (uint32_t)(vcl ^ pf_vswz<D>(vr0))) | (8u * (r16 & 1));
    const uint32_t one2 = BF16 ? 0x3F803F80u : 0x3C003C00u;
    int key_hi = skv - 1, key_lo = 0;
    if (MASK >= kMaskCausal) key_hi = min(key_hi, my_pos);
    if (MASK == kMaskCausalWindow) key_lo = max(key_lo, my_pos - p.window + 1);
    const bool none_visible = key_hi < key_lo;
    const uint32_t key_span = none_visible ? 0u : (uint32_t)(key_hi - key_lo);
    if (none_visible) key_lo = INT_MIN / 2;
    auto mask_half = [&](f32x16& sacc, int kv0, int t) __attribute__((always_inline)) {
        const int base = kv0 + 32 * t + 4 * hf - key_lo;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const uint32_t d = (uint32_t)(base + 8 * (r >> 2) + (r & 3));
            sacc[r] = d <= key_span ? sacc[r] : kMaskedScore;
        }
    };
    auto tile_full = [&](int j) __attribute__((always_inline)) {
        const int kv0 = j * PF_BN;
        bool f = kv0 + PF_BN <= skv;
        if (MASK >= kMaskCausal) f &= kv0 + PF_BN - 1 <= wpos0;
        if (MASK == kMaskCausalWindow) f &= kv0 >= wpos1 - p.window + 1;
        return f;
    };

    constexpr float kLazyRescale = 8.0f;
    float m_i = kMaxInit, l_i = 0.f;
    f32x16 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16{};

    auto tile = [&](int j, int buf) __attribute__((always_inline)) {
        const uint16_t* Kt = Ks[buf];
        f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const uint32_t koff = kfrag ^ (32u * s);
            const s16x8 a0 = *(const s16x8*)((const char*)Kt + koff);
            const s16x8 a1 = *(const s16x8*)((const char*)(Kt + 32 * D) + koff);
            s0 = mfma32x32x16<BF16>(a0, qf[s], s0);
            s1 = mfma32x32x16<BF16>(a1, qf[s], s1);
        }
        if (!(wave_live && tile_full(j))) {
            mask_half(s0, j * PF_BN, 0);
            mask_half(s1, j * PF_BN, 1);
        }
        float mx = kMaskedScore;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = max3f(mx, s0[r], s1[r]);
        mx = max_with_other_half(mx);
        // move m (rescaling O and l) only for rows whose tile max passed m + margin
        const float m_cand = mx * p.c;
        const bool grow = m_cand > m_i + kLazyRescale;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = grow ? m_cand : m_i;
            const float alpha = fast_exp2(m_i - m_new);
            m_i = m_new;
            l_i *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
        }
        const float neg_m = -m_i;
        uint32_t pk[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const f32x16& sc = i < 8 ? s0 : s1;
            const int r = 2 * (i % 8);
            pk[i] = pack2_16<BF16>(fast_exp2(fmaf(sc[r], p.c, neg_m)), fast_exp2(fmaf(sc[r + 1], p.c, neg_m)));
        }
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            ps0 = dot2_16<BF16>(pk[e], one2, ps0);
            ps1 = dot2_16<BF16>(pk[e + 1], one2, ps1);
        }
        l_i += ps0 + ps1;
        const char* Vt = (const char*)Vs[buf];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const s16x8 pb = __builtin_bit_cast(s16x8, make_uint4(pk[4 * u], pk[4 * u + 1], pk[4 * u + 2], pk[4 * u + 3]));
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const char* vb0 = Vt + (vfrag ^ (64u * dt));
                const s16x8 vb = concat4(lds_read_tr16((const uint16_t*)(vb0 + 2 * D * (16 * u))),
                                         lds_read_tr16((const uint16_t*)(vb0 + 2 * D * (16 * u + 8))));
                o[dt] = mfma32x32x16<BF16>(vb, pb, o[dt]);
            }
        }
    };

    if (j_end > j_begin) {
        fetch(j_begin);
        pf_load_q<D>(qf, qrow, my_q < sq, p.qflip);
        store(0);
        __syncthreads();
        for (int j = j_begin; j < j_end; ++j) {
            const int buf = (j - j_begin) & 1;
            const bool more = j + 1 < j_end;
            if (more) fetch(j + 1);
            tile(j, buf);
            // the other buffer was last read in step j - 1, before the barrier that ended it
            if (more) store(buf ^ 1);
            __syncthreads();
        }
    }

    // Epilogue: O * (v_scale / l), with the sink folded in first; rows that saw
    // no key are written as zeros. The log-sum-exp (natural log) goes to lse.
    float l_tot = sum_with_other_half(l_i);
    float m_fin = m_i;
    const float sink = p.sinks ? p.sinks[h] : -__builtin_inff();
    const bool nan_row = sink_gives_nan(sink);
    const float osc = p.sinks ? fold_sink(sink * kLog2e, m_fin, l_tot) : 1.f;
    const float inv = l_tot > 0.f ? osc * p.v_scale / l_tot : 0.f;
    if (p.lse && hf == 0 && wave_live && my_q < sq)
        pf_store_lse(&p.lse[((int64_t)b * p.seqlen_q + my_q) * p.n_q_heads + h], m_fin, l_tot, nan_row);
    pf_store_o16<BF16, NDT>(o, inv,
                            (uint16_t*)p.o + (int64_t)b * p.os.batch + (int64_t)min(my_q, sq - 1) * p.os.seq +
                                (int64_t)h * p.os.head,
                            hf, nan_row, wave_live && my_q < sq);
}

// ---------------------------------------------------------------------------- f32
constexpr int F32_BM = 64;
constexpr int F32_BN = 32;

template <int D, int MASK>
__global__ __launch_bounds__(256) void prefill_f32(PrefillParams p) {
    constexpr int DQ = D / 4;  // dims per lane (four lanes per query row)
    __shared__ __attribute__((aligned(16))) float Ks[F32_BN * D];
    __shared__ __attribute__((aligned(16))) float Vs[F32_BN * D];

    const int tid = threadIdx.x;
    const int r = tid >> 2, qd = tid & 3;
    const int nbh = p.batch * p.n_q_heads;
    const int qt = p.n_q_tiles - 1 - (int)(blockIdx.x / nbh);
    const int bh = blockIdx.x % nbh;
    const int b = bh / p.n_q_heads, h = bh % p.n_q_heads, hk = h / p.group;

    // Sequence b's sizes and the element offsets of its first rows: sequences
    // of one fixed size, or packed sequences delimited by cumulative offsets.
    int sq = p.seqlen_q, skv = p.seqlen_kv;
    int64_t q_at = (int64_t)b * p.qs.batch, k_at = (int64_t)b * p.ks.batch, v_at = (int64_t)b * p.vs.batch,
            o_at = (int64_t)b * p.os.batch, lse_at = (int64_t)b * p.seqlen_q;
    if (p.cu_seqlens_q) {
        const int qs0 = p.cu_seqlens_q[b], ks0 = p.cu_seqlens_kv[b];
        sq = min(p.cu_seqlens_q[b + 1] - qs0, p.seqlen_q);
        skv = p.cu_seqlens_kv[b + 1] - ks0;
        q_at = (int64_t)qs0 * p.qs.seq;
        o_at = (int64_t)qs0 * p.os.seq;
        lse_at = qs0;
        k_at = (int64_t)ks0 * p.ks.seq;
        v_at = (int64_t)ks0 * p.vs.seq;
    }
    const int off = skv - sq;  // query row i sits at position i + off
    const int q0 = qt * F32_BM;
    if (q0 >= sq) return;  // a tile past this sequence's end (packed sequences only)
    const int qlast = min(q0 + F32_BM, sq) - 1;
    // Position of query row i: i + off (bottom-right alignment), or the caller's
    // positions of packed rows (nondecreasing within a sequence).
    auto pos_of = [&](int i) -> int { return p.positions ? p.positions[lse_at + min(i, sq - 1)] : i + off; };
    int kv_lo = 0, kv_hi = skv;
    if (MASK >= kMaskCausal) kv_hi = min(kv_hi, pos_of(qlast) + 1);
    if (MASK == kMaskCausalWindow) kv_lo = max(0, pos_of(q0) - p.window + 1);
    const int j_begin = kv_lo / F32_BN;
    const int j_end = kv_hi > kv_lo ? (kv_hi + F32_BN - 1) / F32_BN : j_begin;

    const int my_q = q0 + r, my_pos = pos_of(my_q);
    const bool live = my_q < sq;
    float qv[DQ], acc[DQ];
    {
        const float* qrow = (const float*)p.q + q_at + (int64_t)my_q * p.qs.seq +
                            (int64_t)h * p.qs.head + qd * DQ;
#pragma unroll
        for (int e = 0; e < DQ; e += 4) {
            float4 x = live ? *(const float4*)(qrow + e) : make_float4(0.f, 0.f, 0.f, 0.f);
            qv[e] = __uint_as_float(__float_as_uint(x.x) ^ p.qflip);
            qv[e + 1] = __uint_as_float(__float_as_uint(x.y) ^ p.qflip);
            qv[e + 2] = __uint_as_float(__float_as_uint(x.z) ^ p.qflip);
            qv[e + 3] = __uint_as_float(__float_as_uint(x.w) ^ p.qflip);
        }
#pragma unroll
        for (int e = 0; e < DQ; ++e) acc[e] = 0.f;
    }
    const float* kbase = (const float*)p.k + k_at + (int64_t)hk * p.ks.head;
    const float* vbase = (const float*)p.v + v_at + (int64_t)hk * p.vs.head;
    float m_i = kMaxInit, l_i = 0.f;

    for (int j = j_begin; j < j_end; ++j) {
        const int kv0 = j * F32_BN;
        __syncthreads();
        for (int c = tid; c < F32_BN * D / 4; c += 256) {
            const int row = c / (D / 4), col = (c % (D / 4)) * 4;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (kv0 + row < skv && kv0 + row >= kv_lo) {
                kx = *(const float4*)(kbase + (int64_t)(kv0 + row) * p.ks.seq + col);
                vx = *(const float4*)(vbase + (int64_t)(kv0 + row) * p.vs.seq + col);
            }
            *(float4*)&Ks[row * D + col] = kx;
            *(float4*)&Vs[row * D + col] = vx;
        }
        __syncthreads();

        float s[F32_BN];
        float mx = kMaskedScore;
#pragma unroll
        for (int kk = 0; kk < F32_BN; ++kk) {
            float part = 0.f;
#pragma unroll
            for (int e = 0; e < DQ; ++e) part = fmaf(qv[e], Ks[kk * D + qd * DQ + e], part);
            part += __shfl_xor(part, 1);
            part += __shfl_xor(part, 2);
            const int key = kv0 + kk;
            bool keep = key < skv;
            if (MASK >= kMaskCausal) keep &= key <= my_pos;
            if (MASK == kMaskCausalWindow) keep &= key >= my_pos - p.window + 1;
            s[kk] = keep ? part : kMaskedScore;
            mx = fmaxf(mx, s[kk]);
        }
        const float m_new = fmaxf(m_i, mx * p.c);
        const float alpha = fast_exp2(m_i - m_new);
        m_i = m_new;
        l_i *= alpha;
#pragma unroll
        for (int e = 0; e < DQ; ++e) acc[e] *= alpha;
#pragma unroll
        for (int kk = 0; kk < F32_BN; ++kk) {
            const float pv = s[kk] == kMaskedScore ? 0.f : fast_exp2(fmaf(s[kk], p.c, -m_new));
            l_i += pv;
#pragma unroll
            for (int e = 0; e < DQ; ++e) acc[e] = fmaf(pv, Vs[kk * D + qd * DQ + e], acc[e]);
        }
    }
    if (live) {
        float m_fin = m_i;
        const float sink = p.sinks ? p.sinks[h] : -__builtin_inff();
        const bool nan_row = sink_gives_nan(sink);
        const float osc = p.sinks ? fold_sink(sink * kLog2e, m_fin, l_i) : 1.f;
        const float inv = l_i > 0.f ? osc / l_i : 0.f;
        if (p.lse && qd == 0) pf_store_lse(&p.lse[(lse_at + my_q) * p.n_q_heads + h], m_fin, l_i, nan_row);
        float* orow = (float*)p.o + o_at + (int64_t)my_q * p.os.seq + (int64_t)h * p.os.head +
                      qd * DQ;
#pragma unroll
        for (int e = 0; e < DQ; e += 4) {
            uint4 bits = make_uint4(__float_as_uint(acc[e] * inv), __float_as_uint(acc[e + 1] * inv),
                                    __float_as_uint(acc[e + 2] * inv), __float_as_uint(acc[e + 3] * inv));
            if (nan_row) bits = make_uint4(kNaN32, kNaN32, kNaN32, kNaN32);
            *(uint4*)(orow + e) = bits;
        }
    }
}

// ---------------------------------------------------------------------------- dispatch
template <bool BF16, int D, int NW, bool KV8 = false>
static hipError_t launch_mfma_nw(PrefillParams p, int mask, hipStream_t s) {
    p.n_q_tiles = (p.seqlen_q + PF_ROWS_PER_WAVE * NW - 1) / (PF_ROWS_PER_WAVE * NW);
    const dim3 grid((unsigned)p.n_q_tiles * p.batch * p.n_q_heads), block(64 * NW);
    switch (mask) {
        case kMaskNone: hipLaunchKernelGGL((prefill_mfma<BF16, D, kMaskNone, NW, KV8>), grid, block, 0, s, p); break;
        case kMaskCausal: hipLaunchKernelGGL((prefill_mfma<BF16, D, kMaskCausal, NW, KV8>), grid, block, 0, s, p); break;
        default: hipLaunchKernelGGL((prefill_mfma<BF16, D, kMaskCausalWindow, NW, KV8>), grid, block, 0, s, p); break;
    }
    return hipGetLastError();
}

// Eight-wave workgroups halve the K/V traffic per FLOP but hold a whole CU
// each; they are used for D <= 128 when there are enough of them to fill the
// chip at least twice over (D = 256 needs more than half a SIMD's registers
// per wave, so it stays at four waves). Packed sequences keep four waves: their
// many short sequences each end in a partly filled tile, and 128-row tiles
// halve that waste (measured 8% faster on 16 prompts of 256..4096 tokens).
constexpr int kPrefillWideMinWorkgroups = 512;

// The persistent D = 256 kernel runs one workgroup per CU (MI355X: 256 CUs, a
// multiple of the 8 XCDs, so every item of a workgroup stays on the XCD the
// plain launch would give it) when there are at least two items per CU, the
// launch is dense with no per-row positions, the mask is a window or none (q
// tiles of like work), and every q tile covers an even number (>= 2) of
// 64-key tiles.
constexpr int kPairItemsWorkgroups = 256;

static bool pair_items_ok(const PrefillShape& s) {
    const int mask = s.mask;
    if (s.packed || s.positions || mask == kMaskCausal || s.seqlen_kv <= 0 || s.seqlen_kv % 64 != 0) return false;
    const int n_q_tiles = (s.seqlen_q + 127) / 128;
    if ((long)n_q_tiles * s.batch * s.n_q_heads < 2L * kPairItemsWorkgroups) return false;
    const int sq = s.seqlen_q, skv = s.seqlen_kv, off = skv - sq;
    // the call's first visible key (the first row's window start) on a tile boundary
    if (mask == kMaskCausalWindow && std::max(0, off - s.window + 1) % 64 != 0) return false;
    for (int t = 0; t < n_q_tiles; ++t) {
        const int q0 = t * 128, qlast = std::min(q0 + 128, sq) - 1;
        int kv_lo = 0, kv_hi = skv;
        if (mask == kMaskCausalWindow) {
            kv_hi = std::min(kv_hi, qlast + off + 1);
            kv_lo = std::max(0, q0 + off - s.window + 1);
        }
        if (kv_hi <= kv_lo) return false;
        const int nt = (kv_hi + 63) / 64 - kv_lo / 64;
        if (nt < 2 || nt % 2 != 0) return false;
    }
    return true;
}

// Eight-wave grids: at least kPrefillWideMinWorkgroups 256-row workgroups.
static bool prefill_wide(const PrefillShape& s) {
    return (long)((s.seqlen_q + 255) / 256) * s.batch * s.n_q_heads >= kPrefillWideMinWorkgroups;
}

int prefill_kernel(const PrefillShape& s) {
    if (s.fp8) return s.head_dim == 128 && prefill_wide(s) ? kPrefillMfma8Kv8 : kPrefillF8kv4;
    if (s.dtype == kF32) return kPrefillF32;
    if (s.head_dim == 256) return pair_items_ok(s) ? kPrefillPairItems : kPrefillPair;
    return !s.packed && prefill_wide(s) ? kPrefillMfma8 : kPrefillMfma4;
}

static PrefillShape shape_of(const PrefillParams& p, int dtype, int head_dim, int mask, bool fp8) {
    return PrefillShape{dtype, fp8, p.cu_seqlens_q != nullptr, p.positions != nullptr, p.batch, p.n_q_heads,
                        p.seqlen_q, p.seqlen_kv, head_dim, mask, p.window};
}

template <bool BF16>
static hipError_t launch_pair(PrefillParams p, bool items, int mask, hipStream_t s) {
    p.n_q_tiles = (p.seqlen_q + 127) / 128;
    if (items) {
        const dim3 grid((unsigned)kPairItemsWorkgroups), block(512);
        if (mask == kMaskCausalWindow)
            hipLaunchKernelGGL((prefill_pair_items<BF16, kMaskCausalWindow>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((prefill_pair_items<BF16, kMaskNone>), grid, block, 0, s, p);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)p.n_q_tiles * p.batch * p.n_q_heads), block(512);
    switch (mask) {
        case kMaskNone: hipLaunchKernelGGL((prefill_pair<BF16, kMaskNone>), grid, block, 0, s, p); break;
        case kMaskCausal: hipLaunchKernelGGL((prefill_pair<BF16, kMaskCausal>), grid, block, 0, s, p); break;
        default: hipLaunchKernelGGL((prefill_pair<BF16, kMaskCausalWindow>), grid, block, 0, s, p); break;
    }
    return hipGetLastError();
}

template <bool BF16, int D>
static hipError_t launch_mfma_mask(PrefillParams p, int kernel, int mask, hipStream_t s) {
    if constexpr (D == 256) {
        return launch_pair<BF16>(p, kernel == kPrefillPairItems, mask, s);
    } else {
        if (kernel == kPrefillMfma8) return launch_mfma_nw<BF16, D, 8>(p, mask, s);
        return launch_mfma_nw<BF16, D, 4>(p, mask, s);
    }
}

template <int D>
static hipError_t launch_f32_mask(PrefillParams p, int mask, hipStream_t s) {
    p.n_q_tiles = (p.seqlen_q + F32_BM - 1) / F32_BM;
    const dim3 grid((unsigned)p.n_q_tiles * p.batch * p.n_q_heads);
    switch (mask) {
        case kMaskNone: hipLaunchKernelGGL((prefill_f32<D, kMaskNone>), grid, dim3(256), 0, s, p); break;
        case kMaskCausal: hipLaunchKernelGGL((prefill_f32<D, kMaskCausal>), grid, dim3(256), 0, s, p); break;
        default: hipLaunchKernelGGL((prefill_f32<D, kMaskCausalWindow>), grid, dim3(256), 0, s, p); break;
    }
    return hipGetLastError();
}

template <bool BF16, int D, int NW>
static hipError_t launch_f8kv_nw(PrefillParams p, int mask, hipStream_t s) {
    p.n_q_tiles = (p.seqlen_q + NW * PF_ROWS_PER_WAVE - 1) / (NW * PF_ROWS_PER_WAVE);
    const dim3 grid((unsigned)p.n_q_tiles * p.batch * p.n_q_heads), block(64 * NW);
    switch (mask) {
        case kMaskNone: hipLaunchKernelGGL((prefill_f8kv<BF16, D, kMaskNone, NW>), grid, block, 0, s, p); break;
        case kMaskCausal: hipLaunchKernelGGL((prefill_f8kv<BF16, D, kMaskCausal, NW>), grid, block, 0, s, p); break;
        default: hipLaunchKernelGGL((prefill_f8kv<BF16, D, kMaskCausalWindow, NW>), grid, block, 0, s, p); break;
    }
    return hipGetLastError();
}

// On the grids where the 16-bit prefill takes eight waves (D = 128), its
// pipelined kernel with FP8 staging; prefill_f8kv otherwise.
template <bool BF16, int D>
static hipError_t launch_f8kv_mask(PrefillParams p, int kernel, int mask, hipStream_t s) {
    if constexpr (D == 128) {
        if (kernel == kPrefillMfma8Kv8) return launch_mfma_nw<BF16, D, 8, true>(p, mask, s);
    }
    return launch_f8kv_nw<BF16, D, 4>(p, mask, s);
}

template <bool BF16>
static hipError_t launch_f8kv_d(const PrefillParams& p, int kernel, int head_dim, int mask, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_f8kv_mask<BF16, 64>(p, kernel, mask, s);
        case 128: return launch_f8kv_mask<BF16, 128>(p, kernel, mask, s);
        default: return launch_f8kv_mask<BF16, 256>(p, kernel, mask, s);
    }
}

hipError_t launch_prefill_f8kv(const PrefillParams& p, int dtype, int head_dim, int mask, hipStream_t s) {
    const int kernel = prefill_kernel(shape_of(p, dtype, head_dim, mask, true));
    return dtype == kBF16 ? launch_f8kv_d<true>(p, kernel, head_dim, mask, s)
                          : launch_f8kv_d<false>(p, kernel, head_dim, mask, s);
}

template <bool BF16>
static hipError_t launch_mfma_d(const PrefillParams& p, int kernel, int head_dim, int mask, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_mfma_mask<BF16, 64>(p, kernel, mask, s);
        case 128: return launch_mfma_mask<BF16, 128>(p, kernel, mask, s);
        default: return launch_mfma_mask<BF16, 256>(p, kernel, mask, s);
    }
}

hipError_t launch_prefill(const PrefillParams& p, int dtype, int head_dim, int mask, hipStream_t s) {
    const int kernel = prefill_kernel(shape_of(p, dtype, head_dim, mask, false));
    if (kernel == kPrefillF32) {
        switch (head_dim) {
            case 64: return launch_f32_mask<64>(p, mask, s);
            case 128: return launch_f32_mask<128>(p, mask, s);
            default: return launch_f32_mask<256>(p, mask, s);
        }
    }
    return dtype == kBF16 ? launch_mfma_d<true>(p, kernel, head_dim, mask, s)
                          : launch_mfma_d<false>(p, kernel, head_dim, mask, s);
}

}  // namespace attn
