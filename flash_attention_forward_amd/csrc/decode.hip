// Split-KV decode attention and the log-sum-exp combine for gfx950.
//
// decode_split: one wavefront per (split, kv-head, sequence), HW of them (the
// kv-heads of one split) per workgroup, so that the rows of all heads of a
// page are read by one CU at about the same time. The G * s_active
// query rows that share a kv-head (G = n_q_heads / n_kv_heads) ride one MFMA
// together, so each K/V byte is read once for all of them — the decode page's
// grouped-query "free broadcast" ("Flash-Attention: Decode (TKG)", section
// "GQA / MQA grouped-query broadcast"), done here with v_mfma_f32_16x16x32
// (16 key rows x 16 query columns, query columns beyond G * s_active are
// zero). Keys are gathered through the uint32 page table, 32 per iteration
// (decode page, section "Paged / block cache"): whole 256-byte K and V rows
// are loaded straight into LDS, K read back as the MFMA A operand and V read
// back transposed with ds_read_b64_tr_b16 for O^T += V^T P^T. The next 32 keys
// are in flight while the current ones are used. All loads go to LDS, so the
// only waits on them are the explicit per-block ones. Rows at or beyond
// cache_len are never read (decode page, section "gen_mask_tkg": index <
// cache length): their loads are clamped to the last valid row, whose copy
// gets probability exactly 0, so nothing past the end can leak into the
// product.
//
// decode_split_f8: the same split for an FP8 E4M3 cache, read into registers
// with full-row loads and widened exactly to 16 bits before the same MFMAs.
//
// Each split writes its normalised output and its natural-log log-sum-exp
// (the decode page's deferred normalisation on its flash path: the partial
// output plus the statistics needed to merge it later).
//
// decode_combine: per (sequence, query, q-head), M = max_s lse_s,
// w_s = exp(lse_s - M), O = sum_s w_s O_s / sum_s w_s (M kept as a running
// maximum over rounds of splits, rescaling what was summed before) — the CTE page's
// cross-section merge (section "Algorithm — running-sum update, reciprocal,
// output accumulate") over any number of splits.
#include <algorithm>
#include <mutex>

#include "attn.h"
#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {

constexpr int DC_KB = 32;   // keys per iteration: two 16-key MFMA row blocks

__device__ __forceinline__ float max_over_groups(float x) {
    // max over the four 16-lane groups, for every lane
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    return max_with_other_half(x);
}
__device__ __forceinline__ float sum_over_groups(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    return sum_with_other_half(x);
}

// Running max in scaled log2 units. It only moves when a row's block max
// exceeds it by more than kDecodeLazyRescale, so O and l are rescaled rarely
// (a wave-uniform branch); in between, probabilities are at most
// 2^kDecodeLazyRescale, and the normalised result is the same softmax.
constexpr float kDecodeLazyRescale = 8.0f;

// Online-softmax update for one 32-key block of S^T (lane (n, g) holds keys
// tb + 16 gi + 4 g + r of query row n, raw scores): moves m_i (rescaling l_i
// and O when it moves) and returns this lane's P^T as the B operand of
// O^T += V^T P^T (slot j of group g is key 4g + j for j < 4, else 16 + 4g + j - 4).
// MASKED applies the visibility cut t < t1, t <= qpos (and the window); a
// block that every row of the wave sees in full skips it. Hidden scores get
// probability exactly 0 and never move m.
template <bool BF16, bool MASKED, int NDT>
__device__ __forceinline__ s16x8 dc_block_probs(f32x4 (&sacc)[2], f32x4 (&o)[NDT], float& m_i, float& l_i, float c,
                                                int tb, int g, int t1, int qpos, int window) {
    float mx = kMaskedScore;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (MASKED) {
                const int t = tb + 16 * gi + 4 * g + r;
                bool keep = t < t1 && t <= qpos;
                if (window > 0) keep &= t >= qpos - window + 1;
                sacc[gi][r] = keep ? sacc[gi][r] : kMaskedScore;
            }
            mx = fmaxf(mx, sacc[gi][r]);
        }
    mx = max_over_groups(mx);
    const float m_cand = mx * c;
    const bool grow = m_cand > m_i + kDecodeLazyRescale;
    if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? m_cand : m_i;
        const float alpha = fast_exp2(m_i - m_new);
        m_i = m_new;
        l_i *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
    }
    const uint32_t one2 = BF16 ? 0x3F803F80u : 0x3C003C00u;  // two 16-bit 1.0s for the row-sum dot2
    uint32_t pk[4];
    float psum = 0.f;
#pragma unroll
    for (int jj = 0; jj < 8; jj += 2) {
        const float s0 = sacc[jj >> 2][jj & 3], s1 = sacc[jj >> 2][(jj & 3) + 1];
        float p0 = fast_exp2(fmaf(s0, c, -m_i)), p1 = fast_exp2(fmaf(s1, c, -m_i));
        if constexpr (MASKED) {
            // (with the smallest scales, mask * c need not underflow to 0)
            p0 = s0 == kMaskedScore ? 0.f : p0;
            p1 = s1 == kMaskedScore ? 0.f : p1;
        }
        pk[jj / 2] = pack2_16<BF16>(p0, p1);
        psum = dot2_16<BF16>(pk[jj / 2], one2, psum);
    }
    l_i += psum;
    return __builtin_bit_cast(s16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
}

// 16-byte chunk swizzle of a V row in LDS: chunk c of row r lives at c ^ f(r).
// With it the 32 lanes of a transpose read (8 rows x two adjacent chunks) hit
// 16 distinct bank groups, while each direct-to-LDS load still fills whole rows.
template <int D>
__device__ __forceinline__ int dc_vswz(int row) {
    return D == 64 ? 2 * ((row >> 1) & 3) : 2 * (row & 7);
}

// FLAT: contiguous cache. FAST: pages of a power-of-two size >= 16, so that
// every 16-key group of a block lies in one page and needs one (uniform)
// lookup. GENERIC: any page size; one lookup per key row.
enum DecodeMode { kDecodeFlat = 0, kDecodeFast = 1, kDecodeGeneric = 2 };

// Kv-heads (waves) per workgroup: each wave holds 32 KB * D / 128 of LDS.
// Four heads (128 KB at D = 128, one workgroup per CU) read 1 KB of each
// token row of the paged workload together and measured 3% faster than two
// with long splits (4096 tokens), 5% slower with short ones (1024), whose
// workgroups are too short-lived to hide their start-up alone on a CU.
template <int D>
constexpr int dc_max_heads() {
    return D >= 256 ? 1 : 4;
}
// decode_split_f8 holds one 16-bit V tile and one byte K tile per wave (12 KB *
// D / 128). Eight kv-heads (97 KB at D = 128, one workgroup per CU) read each
// token's whole row of the paged FP8 workload (1 KB) together; four (two
// workgroups per CU) read it in two halves. Eight measured 5-7% faster with
// 1792- to 2048-token splits on the paged workload and 8% slower with
// 512-token splits, so the launch takes eight only on grids of at least
// kDecodeF8WideGrid workgroups (with fewer, eight-wave workgroups leave CUs
// idle). D = 256 holds two.
template <int D>
constexpr int dc_max_heads_f8() {
    return D >= 256 ? 2 : 8;
}
constexpr int64_t kDecodeF8WideGrid = 512;

// 16-byte chunk swizzle of a K row in LDS: the 16 lanes of a fragment read hit
// rows r..r+15 at one chunk, spread over 16 bank groups.
template <int D>
__device__ __forceinline__ int dc_kswz(int row) {
    return D == 64 ? ((row >> 1) & 7) : (row & 15);
}

template <bool BF16, int D, int MODE, int HW, int QB>
__global__ __launch_bounds__(64 * HW) void decode_split(DecodeParams p) {
    constexpr int NKS = D / 32;              // k-steps of S^T = K Q^T
    constexpr int NDT = D / 16;              // 16-row d tiles of O^T
    constexpr int CPR = D / 8;               // 16-byte chunks per V row
    constexpr int RPL = 64 / CPR;            // V rows covered by one direct-to-LDS load
    constexpr int VLD = DC_KB / RPL;         // direct-to-LDS loads per lane per block and tensor
    // Two K and two V tiles per wave in LDS: block i+2 is requested while
    // block i is used, so each block's loads have a whole iteration to land.
    // The tiles are private to their wave.
    __shared__ __attribute__((aligned(16))) uint16_t KsA[HW][DC_KB * D];
    __shared__ __attribute__((aligned(16))) uint16_t KsB[HW][DC_KB * D];
    __shared__ __attribute__((aligned(16))) uint16_t VsA[HW][DC_KB * D];
    __shared__ __attribute__((aligned(16))) uint16_t VsB[HW][DC_KB * D];
    // This split's slice of the page table, read once: address generation in
    // the loop then never waits on a global load.
    __shared__ uint32_t pages[kDecodeMaxSplitPages];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // wave index, uniform
    const int n = lane & 15;   // query column / key row within a 16-block
    const int g = lane >> 4;   // 16-lane group
    const int hk = blockIdx.x * HW + w, split = blockIdx.y, b = blockIdx.z;

    const int t0 = split * p.split_len;
    // Query rows (G * s_active of them) ride the 16 MFMA columns, in QB blocks
    // of 16: block qb, column n is row 16 qb + n.
    const int nrows = p.group * p.s_active;
    bool row_real[QB];
    int qi[QB], qh[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = 16 * qb + n;
        row_real[qb] = row < nrows;
        qi[qb] = row_real[qb] ? row / p.group : 0;
        qh[qb] = hk * p.group + (row_real[qb] ? row % p.group : 0);
    }

    // Requested together before anything waits: cache_len[b], this split's
    // whole slice of the page table (clamped to the table row; entries past
    // the cache are never used) and the Q fragments.
    constexpr int PPT = (kDecodeMaxSplitPages + 64 * HW - 1) / (64 * HW);  // page entries per thread
    uint32_t pe[PPT];
    const int spp = MODE == kDecodeFlat ? 0 : p.split_len / p.page_size;  // pages per split, <= 256
    if constexpr (MODE != kDecodeFlat) {
        const uint32_t* trow = p.block_table + (int64_t)b * p.max_pages_per_seq;
        const int first = t0 / p.page_size, last = p.max_pages_per_seq - 1;
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int i = (int)threadIdx.x + k * 64 * HW;
            pe[k] = i < spp && last >= 0 ? trow[min(first + i, last)] : 0u;
        }
    }
    // Q fragments: B operand of S^T = K Q^T (lane: column n, d = 32ks + 8g .. +8).
    s16x8 qf[QB][NKS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const uint16_t* qrow = (const uint16_t*)p.q + (int64_t)b * p.qs.batch + (int64_t)qi[qb] * p.qs.seq +
                               (int64_t)qh[qb] * p.qs.head + 8 * g;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (row_real[qb]) x = *(const uint4*)(qrow + 32 * ks);
            x.x ^= p.qflip; x.y ^= p.qflip; x.z ^= p.qflip; x.w ^= p.qflip;
            qf[qb][ks] = __builtin_bit_cast(s16x8, x);
        }
    }
    const int len = p.cache_len[b];
    if (t0 >= len) return;  // this split is past the cache: nothing is written (uniform in the workgroup)
    const int t1 = min(len, t0 + p.split_len);
    int qpos[QB];      // the queries sit at the end of their cache
    int64_t prow[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        qpos[qb] = len - p.s_active + qi[qb];
        prow[qb] = (((int64_t)b * p.s_active + qi[qb]) * p.n_q_heads + qh[qb]) * p.max_splits + split;
    }

    // Keys this split may use: [t0, t1) clipped to the window of the earliest query.
    int tlo = t0;
    if (p.window > 0) tlo = max(tlo, (len - p.s_active) - p.window + 1);
    if (tlo >= t1) {  // no visible key: empty partial
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            if (!row_real[qb]) continue;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                *(float4*)(p.part_o + prow[qb] * D + 16 * dt + 4 * g) = make_float4(0.f, 0.f, 0.f, 0.f);
            if (g == 0) p.part_lse[prow[qb]] = -__builtin_inff();
        }
        return;
    }
    const int tb0 = t0 + ((tlo - t0) / DC_KB) * DC_KB;  // first iteration's key block
    const int nblk = (t1 - tb0 + DC_KB - 1) / DC_KB;
    if constexpr (MODE != kDecodeFlat) {
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int i = (int)threadIdx.x + k * 64 * HW;
            if (i < spp) pages[i] = pe[k];
        }
        __syncthreads();  // the only workgroup barrier: every early return above is uniform
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // from here on vmcnt counts K/V block loads only

    const uint16_t* kbase = (const uint16_t*)p.k + (int64_t)hk * p.kvs.head;
    const uint16_t* vbase = (const uint16_t*)p.v + (int64_t)hk * p.kvs.head;
    const int64_t seq = p.kvs.seq;
    // Element offset of token t's row (GENERIC, and the first row of a 16-key group in FAST).
    auto row_off = [&](int t) -> int64_t {
        if constexpr (MODE == kDecodeFlat) {
            return (int64_t)b * p.kvs.batch + (int64_t)t * seq;
        } else {
            const int rel = t - t0;
            int pi, slot;
            if constexpr (MODE == kDecodeFast) {
                pi = rel >> p.page_shift;
                slot = rel & (p.page_size - 1);
            } else {
                pi = rel / p.page_size;
                slot = rel - pi * p.page_size;
            }
            return (int64_t)pages[pi] * p.kvs.batch + (int64_t)slot * seq;
        }
    };

    // Every load is issued unconditionally with its row clamped to a valid
    // token: rows past the end (and whole blocks past the last one), and rows
    // of the first block below the earliest query's window, re-read cache
    // data that some query row sees, get probability exactly 0 in the softmax
    // and so add exactly nothing to P V. Nothing at or beyond cache_len and
    // nothing before that window is ever read. With
    // no conditional loads, each lane has exactly 2 * VLD loads per block in
    // flight and the wait counts below hold on every path.
    const int tlast = t1 - 1;
    // Keys in [t_from, t_full) are visible to every query row of the wave.
    const int t_full = min(t1, len - p.s_active + 1);
    const int t_from = p.window > 0 ? len - p.window : 0;
    // FAST: offset of the 16-aligned group holding token t, plus the row within it
    auto fast_off = [&](int t) -> int64_t {
        const int tc = min(max(t, tlo), tlast);
        const int tg = tc & ~15;
        return row_off(tg) + (int64_t)(tc - tg) * seq;
    };
    // Element offset of the first row of the 16-key group at tg (FLAT, FAST), as a wave-uniform value.
    auto group_off = [&](int tg) -> int64_t {
        if constexpr (MODE == kDecodeFlat) {
            return (int64_t)b * p.kvs.batch + (int64_t)tg * seq;
        } else {
            const int rel = tg - t0;
            const uint32_t page = __builtin_amdgcn_readfirstlane(pages[rel >> p.page_shift]);
            return (int64_t)page * p.kvs.batch + (int64_t)(rel & (p.page_size - 1)) * seq;
        }
    };
    // A K or V block straight into LDS: load i writes LDS bytes [1 KB * i,
    // 1 KB * (i + 1)), lane L landing at row i * RPL + L / CPR, swizzled chunk L % CPR.
    // The cache is read once, so the loads are non-temporal (the nt cache
    // policy): the stream does not push the partials and the page table out
    // of L2, and measured 4-6% faster than default-policy loads.
    constexpr int kStreamPolicy = 2;  // nt
    const int cs = lane % CPR;
    // A block that ends before t1 (in FLAT and FAST mode) is addressed as a
    // wave-uniform base per 16-key group (page entry, slot: scalar
    // arithmetic) plus a per-lane byte offset fixed for the whole loop (row
    // within the group, swizzled chunk), so its loads cost no vector ALU work.
    const bool lane_addr = MODE != kDecodeGeneric && p.lane_addr32;
    auto load_rows = [&](uint16_t* dst, const uint16_t* base, int tb, bool is_k) __attribute__((always_inline)) {
        if (lane_addr && tb >= tlo && tb + DC_KB <= t1) {
            const int64_t g0 = group_off(tb), g1 = group_off(tb + 16);
#pragma unroll
            for (int i = 0; i < VLD; ++i) {
                // (loop-invariant: computed once, outside the key loop)
                const int row = i * RPL + lane / CPR;
                const int c = cs ^ (is_k ? dc_kswz<D>(row) : dc_vswz<D>(row));
                const uint32_t lane_off = (uint32_t)(((row & 15) * seq + 8 * c) * 2);
                const char* gb = (const char*)(base + (i * RPL < 16 ? g0 : g1));
                __builtin_amdgcn_global_load_lds(gb + lane_off,
                                                 (__attribute__((address_space(3))) void*)(dst + 512 * i), 16, 0,
                                                 kStreamPolicy);
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int row = i * RPL + lane / CPR;
            const int t = tb + row;
            const int c = cs ^ (is_k ? dc_kswz<D>(row) : dc_vswz<D>(row));
            const int64_t off = MODE == kDecodeGeneric ? row_off(min(max(t, tlo), tlast)) : fast_off(t);
            __builtin_amdgcn_global_load_lds(base + off + 8 * c, (__attribute__((address_space(3))) void*)(dst + 512 * i),
                                             16, 0, kStreamPolicy);
        }
    };
    float m_i[QB], l_i[QB];
    f32x4 o[QB][NDT];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_i[qb] = kMaxInit;
        l_i[qb] = 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[qb][dt] = f32x4{};
    }

    // One block: wait for its loads, S^T = K Q^T, refill these K registers with
    // block it+2, online softmax, O^T += V^T P^T, refill this V tile with block it+2.
    auto step = [&](uint16_t* K, uint16_t* V, int it) {
        const int tb = tb0 + it * DC_KB;
        wait_vmcnt<2 * VLD>();  // only block it+1's loads may still be in flight

        // S^T = K Q^T: lane (n, g) reads key row 16gi + n, d chunk 4ks + g.
        f32x4 sacc[QB][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[qb][0] = sacc[qb][1] = f32x4{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) {
                const int row = 16 * gi + n;
                const s16x8 a = *(const s16x8*)&K[row * D + 8 * ((4 * ks + g) ^ dc_kswz<D>(row))];
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sacc[qb][gi] = mfma16x16x32<BF16>(a, qf[qb][ks], sacc[qb][gi]);
            }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // K fragment reads done before the tile is refilled
        load_rows(K, kbase, tb + 2 * DC_KB, true);  // block it+2 (clamped rows when past the end)

        // rows at or beyond t1 hold another row's keys: masked in the edge blocks
        const bool full = tb + DC_KB <= t_full && tb >= t_from;
        s16x8 pb[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            pb[qb] = full ? dc_block_probs<BF16, false>(sacc[qb], o[qb], m_i[qb], l_i[qb], p.c, tb, g, t1, qpos[qb],
                                                        p.window)
                          : dc_block_probs<BF16, true>(sacc[qb], o[qb], m_i[qb], l_i[qb], p.c, tb, g, t1, qpos[qb],
                                                       p.window);

        // O^T[d, q] += V^T[d, keys] P^T[keys, q]; lane n of group g reads rows
        // 4g + n/4 (and 16 + ...), column 16dt + 4(n%4), receiving column 16dt + n.
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int c = 2 * dt + ((n & 3) >> 1), half = 4 * (n & 1);
            const int r0 = 4 * g + (n >> 2), r1 = r0 + 16;
            const s16x4 lo = lds_read_tr16(&V[r0 * D + 8 * (c ^ dc_vswz<D>(r0)) + half]);
            const s16x4 hi4 = lds_read_tr16(&V[r1 * D + 8 * (c ^ dc_vswz<D>(r1)) + half]);
            const s16x8 vf = concat4(lo, hi4);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) o[qb][dt] = mfma16x16x32<BF16>(vf, pb[qb], o[qb][dt]);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // transpose reads done before the tile is refilled
        load_rows(V, vbase, tb + 2 * DC_KB, false);
    };

    load_rows(KsA[w], kbase, tb0, true);
    load_rows(VsA[w], vbase, tb0, false);
    load_rows(KsB[w], kbase, tb0 + DC_KB, true);
    load_rows(VsB[w], vbase, tb0 + DC_KB, false);
    // An odd block count runs one extra, fully masked block (no loads beyond the clamp).
    for (int it = 0; it < nblk; it += 2) {
        step(KsA[w], VsA[w], it);
        step(KsB[w], VsB[w], it + 1);
    }
    wait_vmcnt<0>();  // drain the clamped prefetches before the wave ends

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l_tot = sum_over_groups(l_i[qb]);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        if (row_real[qb]) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                *(float4*)(p.part_o + prow[qb] * D + 16 * dt + 4 * g) =
                    make_float4(o[qb][dt][0] * inv, o[qb][dt][1] * inv, o[qb][dt][2] * inv, o[qb][dt][3] * inv);
            if (g == 0)
                p.part_lse[prow[qb]] =
                    l_tot > 0.f ? (m_i[qb] + __log2f(l_tot)) * 0.69314718055994531f : -__builtin_inff();
        }
    }
}

// decode_split_f8: decode_split for a K/V cache stored in FP8 E4M3 (the OCP
// "fn" encoding; the decode page's FP8-e4m3 KV cache), with q, the partials
// and the output as in decode_split. A stored code stands for k_scale (or
// v_scale) times its value; k_scale is folded into the softmax scale on the
// host and v_scale multiplies each split's output. The codes are widened
// exactly to bf16 (gfx950's v_cvt_scalef32_pk_bf16_fp8, scale 1) and the
// products run on the same bf16/f16 MFMAs, so the only rounding beyond the
// 16-bit path is the cache's own.
//
// Cache reads are plain 16-byte register loads (non-temporal), so the
// compiler's own wait counting covers them exactly. Each load instruction
// reads whole rows: D/16 consecutive lanes cover one row, so a 128-byte row
// is one full-line request (a CU keeps a bounded number of requests in
// flight, so half-line requests would halve the bytes in flight). Two
// register sets alternate: a set is refilled with block i+2 as soon as block
// i's codes have gone to LDS, so two blocks are in flight while block i is
// multiplied. K's codes go to a per-wave byte tile, read back in the MFMA
// A-operand layout with a permuted d order: lane (n, g) takes row n of a
// 16-key group and bytes [64 j + 16 g, +16) of it, so k-step ks of the
// product uses d = 64 (ks/2) + 16 g + 8 (ks%2) .. +8; Q's B operand uses the
// same order, so the sum over d is unchanged. V is widened in registers and
// written as bf16 rows into the wave's V tile (decode_split's layout and
// swizzle), from which the transpose reads build V^T.
template <int D>
__device__ __forceinline__ int dc_kcswz(int row) {
    // 16-byte chunk swizzle of the K code tile: the 16 lanes of an operand
    // read (rows r..r+15, one chunk) hit distinct bank groups.
    return D == 64 ? ((row >> 1) & 3) : (row & 7);
}

template <bool BF16, int D, int MODE, int HW, int QB>
__global__ __launch_bounds__(64 * HW) void decode_split_f8(DecodeParams p) {
    constexpr int NKS = D / 32;   // k-steps of S^T = K Q^T
    constexpr int NDT = D / 16;   // 16-row d tiles of O^T
    constexpr int NLD = D / 64;   // 16-byte operand reads per lane and 16-key group
    constexpr int CPR = D / 16;   // 16-byte code chunks per row (= lanes per row in a load)
    constexpr int RPI = 64 / CPR; // rows per load instruction
    constexpr int NI = DC_KB / RPI;  // load instructions per block and tensor
    static_assert(NLD >= 1 && RPI <= 16, "D in 64..256");
    __shared__ __attribute__((aligned(16))) uint16_t Vs[HW][DC_KB * D];
    __shared__ __attribute__((aligned(16))) uint8_t Kc[HW][DC_KB * D];
    __shared__ uint32_t pages[kDecodeMaxSplitPages];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int n = lane & 15;
    const int g = lane >> 4;
    const int hk = blockIdx.x * HW + w, split = blockIdx.y, b = blockIdx.z;

    const int t0 = split * p.split_len;
    // Query rows (G * s_active of them) ride the 16 MFMA columns, in QB blocks
    // of 16: block qb, column n is row 16 qb + n.
    const int nrows = p.group * p.s_active;
    bool row_real[QB];
    int qi[QB], qh[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = 16 * qb + n;
        row_real[qb] = row < nrows;
        qi[qb] = row_real[qb] ? row / p.group : 0;
        qh[qb] = hk * p.group + (row_real[qb] ? row % p.group : 0);
    }

    constexpr int PPT = (kDecodeMaxSplitPages + 64 * HW - 1) / (64 * HW);
    uint32_t pe[PPT];
    const int spp = MODE == kDecodeFlat ? 0 : p.split_len / p.page_size;
    if constexpr (MODE != kDecodeFlat) {
        const uint32_t* trow = p.block_table + (int64_t)b * p.max_pages_per_seq;
        const int first = t0 / p.page_size, last = p.max_pages_per_seq - 1;
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int i = (int)threadIdx.x + k * 64 * HW;
            pe[k] = i < spp && last >= 0 ? trow[min(first + i, last)] : 0u;
        }
    }
    // Q fragments in the permuted d order: lane (n, g), k-step ks holds d = 64 (ks/2) + 16 g + 8 (ks%2) .. +8.
    s16x8 qf[QB][NKS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const uint16_t* qrow = (const uint16_t*)p.q + (int64_t)b * p.qs.batch + (int64_t)qi[qb] * p.qs.seq +
                               (int64_t)qh[qb] * p.qs.head + 16 * g;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (row_real[qb]) x = *(const uint4*)(qrow + 64 * (ks / 2) + 8 * (ks % 2));
            x.x ^= p.qflip; x.y ^= p.qflip; x.z ^= p.qflip; x.w ^= p.qflip;
            qf[qb][ks] = __builtin_bit_cast(s16x8, x);
        }
    }
    const int len = p.cache_len[b];
    if (t0 >= len) return;
    const int t1 = min(len, t0 + p.split_len);
    int qpos[QB];
    int64_t prow[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        qpos[qb] = len - p.s_active + qi[qb];
        prow[qb] = (((int64_t)b * p.s_active + qi[qb]) * p.n_q_heads + qh[qb]) * p.max_splits + split;
    }

    int tlo = t0;
    if (p.window > 0) tlo = max(tlo, (len - p.s_active) - p.window + 1);
    if (tlo >= t1) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            if (!row_real[qb]) continue;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                *(float4*)(p.part_o + prow[qb] * D + 16 * dt + 4 * g) = make_float4(0.f, 0.f, 0.f, 0.f);
            if (g == 0) p.part_lse[prow[qb]] = -__builtin_inff();
        }
        return;
    }
    const int tb0 = t0 + ((tlo - t0) / DC_KB) * DC_KB;
    const int nblk = (t1 - tb0 + DC_KB - 1) / DC_KB;
    if constexpr (MODE != kDecodeFlat) {
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int i = (int)threadIdx.x + k * 64 * HW;
            if (i < spp) pages[i] = pe[k];
        }
        __syncthreads();
    }
    // Q, cache_len and the page table are in: from here on the only loads in
    // flight are cache blocks, so the compiler's wait counts in the loop are exact.
    wait_vmcnt<0>();

    const uint8_t* kbase = (const uint8_t*)p.k + (int64_t)hk * p.kvs.head;
    const uint8_t* vbase = (const uint8_t*)p.v + (int64_t)hk * p.kvs.head;
    const int64_t seq = p.kvs.seq;
    auto row_off = [&](int t) -> int64_t {
        if constexpr (MODE == kDecodeFlat) {
            return (int64_t)b * p.kvs.batch + (int64_t)t * seq;
        } else {
            const int rel = t - t0;
            int pi, slot;
            if constexpr (MODE == kDecodeFast) {
                pi = rel >> p.page_shift;
                slot = rel & (p.page_size - 1);
            } else {
                pi = rel / p.page_size;
                slot = rel - pi * p.page_size;
            }
            return (int64_t)pages[pi] * p.kvs.batch + (int64_t)slot * seq;
        }
    };
    // Rows are clamped to [tlo, t1) (see decode_split): rows past the end and
    // below the earliest query's window re-read visible cache data and get
    // probability exactly 0.
    const int tlast = t1 - 1;
    // Keys in [t_from, t_full) are visible to every query row of the wave.
    const int t_full = min(t1, len - p.s_active + 1);
    const int t_from = p.window > 0 ? len - p.window : 0;
    auto tok_off = [&](int t) -> int64_t {
        const int tc = min(max(t, tlo), tlast);
        if constexpr (MODE == kDecodeFast) {
            const int tg = tc & ~15;
            return row_off(tg) + (int64_t)(tc - tg) * seq;
        } else {
            return row_off(tc);
        }
    };
    // Byte offset of the first row of the 16-key group at tg (FLAT, FAST), as a wave-uniform value.
    auto group_off = [&](int tg) -> int64_t {
        if constexpr (MODE == kDecodeFlat) {
            return (int64_t)b * p.kvs.batch + (int64_t)tg * seq;
        } else {
            const int rel = tg - t0;
            const uint32_t page = __builtin_amdgcn_readfirstlane(pages[rel >> p.page_shift]);
            return (int64_t)page * p.kvs.batch + (int64_t)(rel & (p.page_size - 1)) * seq;
        }
    };
    // Load i of a block: lane L takes row RPI i + L / CPR, bytes [16 (L % CPR), +16).
    const int lrow = lane / CPR, lchunk = lane % CPR;
    // A block that ends before t1 (FLAT, FAST) is addressed as that uniform
    // base plus this lane's fixed offset, so its loads cost no vector ALU
    // work; other blocks clamp row by row.
    const bool lane_addr = MODE != kDecodeGeneric && p.lane_addr32;
    auto load_block = [&](uint4 (&kr)[NI], uint4 (&vr)[NI], int tb) __attribute__((always_inline)) {
        if (lane_addr && tb >= tlo && tb + DC_KB <= t1) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int64_t go = group_off(tb + ((RPI * i) & ~15));
                const uint32_t lo = (uint32_t)(((RPI * i) % 16 + lrow) * seq + 16 * lchunk);
                kr[i] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)(kbase + go + lo)));
                vr[i] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)(vbase + go + lo)));
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int64_t off = tok_off(tb + RPI * i + lrow) + 16 * lchunk;
            kr[i] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)(kbase + off)));
            vr[i] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)(vbase + off)));
        }
    };
    // 8 codes (two dwords, low byte first) -> 8 values of the product's 16-bit type as one MFMA
    // operand (exact: every E4M3 value is a bf16 and an f16 value).
    auto operand8 = [](uint32_t lo, uint32_t hi) __attribute__((always_inline)) {
        uint32_t w[4];
        if constexpr (BF16) {
            w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
            w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
            w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
            w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
        } else {
            w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false));
            w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true));
            w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false));
            w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true));
        }
        return __builtin_bit_cast(s16x8, make_uint4(w[0], w[1], w[2], w[3]));
    };

    float m_i[QB], l_i[QB];
    f32x4 o[QB][NDT];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_i[qb] = kMaxInit;
        l_i[qb] = 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[qb][dt] = f32x4{};
    }
    uint16_t* V = Vs[w];
    uint8_t* K = Kc[w];

    auto step = [&](uint4 (&kr)[NI], uint4 (&vr)[NI], int it) {
        const int tb = tb0 + it * DC_KB;
        // (the fence keeps the scheduler from hoisting this block's code,
        // whose loads were issued one step ago, into the previous step)
        sched_fence();
        // K codes to the byte tile, V rows widened into the bf16 tile (chunks 2c, 2c + 1)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int row = RPI * i + lrow;
            *(uint4*)&K[row * D + 16 * (lchunk ^ dc_kcswz<D>(row))] = kr[i];
            const s16x8 lo8 = operand8(vr[i].x, vr[i].y), hi8 = operand8(vr[i].z, vr[i].w);
            *(s16x8*)&V[row * D + 8 * ((2 * lchunk) ^ dc_vswz<D>(row))] = lo8;
            *(s16x8*)&V[row * D + 8 * ((2 * lchunk + 1) ^ dc_vswz<D>(row))] = hi8;
        }
        load_block(kr, vr, tb + 2 * DC_KB);  // this set now carries block it+2 (clamped past the end)

        // S^T = K Q^T from the code tile (one wave's own LDS writes are seen by its later reads)
        f32x4 sacc[QB][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[qb][0] = sacc[qb][1] = f32x4{};
#pragma unroll
        for (int j = 0; j < NLD; ++j)
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) {
                const int row = 16 * gi + n;
                const uint4 c4 = *(const uint4*)&K[row * D + 16 * ((4 * j + g) ^ dc_kcswz<D>(row))];
                const s16x8 a0 = operand8(c4.x, c4.y), a1 = operand8(c4.z, c4.w);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    sacc[qb][gi] = mfma16x16x32<BF16>(a0, qf[qb][2 * j], sacc[qb][gi]);
                    sacc[qb][gi] = mfma16x16x32<BF16>(a1, qf[qb][2 * j + 1], sacc[qb][gi]);
                }
            }
        const bool full = tb + DC_KB <= t_full && tb >= t_from;
        s16x8 pb[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            pb[qb] = full ? dc_block_probs<BF16, false>(sacc[qb], o[qb], m_i[qb], l_i[qb], p.c, tb, g, t1, qpos[qb],
                                                        p.window)
                          : dc_block_probs<BF16, true>(sacc[qb], o[qb], m_i[qb], l_i[qb], p.c, tb, g, t1, qpos[qb],
                                                       p.window);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int c = 2 * dt + ((n & 3) >> 1), half = 4 * (n & 1);
            const int r0 = 4 * g + (n >> 2), r1 = r0 + 16;
            const s16x4 lo = lds_read_tr16(&V[r0 * D + 8 * (c ^ dc_vswz<D>(r0)) + half]);
            const s16x4 hi4 = lds_read_tr16(&V[r1 * D + 8 * (c ^ dc_vswz<D>(r1)) + half]);
            const s16x8 vf = concat4(lo, hi4);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) o[qb][dt] = mfma16x16x32<BF16>(vf, pb[qb], o[qb][dt]);
        }
    };

    uint4 kA[NI], vA[NI], kB[NI], vB[NI];
    load_block(kA, vA, tb0);
    load_block(kB, vB, tb0 + DC_KB);
    for (int it = 0; it < nblk; it += 2) {
        step(kA, vA, it);
        step(kB, vB, it + 1);
    }
    wait_vmcnt<0>();

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l_tot = sum_over_groups(l_i[qb]);
        const float inv = l_tot > 0.f ? p.v_scale / l_tot : 0.f;
        if (row_real[qb]) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                *(float4*)(p.part_o + prow[qb] * D + 16 * dt + 4 * g) =
                    make_float4(o[qb][dt][0] * inv, o[qb][dt][1] * inv, o[qb][dt][2] * inv, o[qb][dt][3] * inv);
            if (g == 0)
                p.part_lse[prow[qb]] =
                    l_tot > 0.f ? (m_i[qb] + __log2f(l_tot)) * 0.69314718055994531f : -__builtin_inff();
        }
    }
}

// One wave per output row. A split's partial row is read as float4s by
// D / 4 lanes, so one load instruction covers 64 / (D / 4) splits; up to 32
// instructions per lane are issued together with the matching log-sum-exps,
// whose maximum is taken while the rows are in flight. The lane groups that
// took different splits are summed with lane swaps at the end.
template <bool BF16, int D>
__global__ __launch_bounds__(64) void decode_combine(CombineParams p) {
    constexpr int LPR = D / 4;      // lanes per split row
    constexpr int RPW = 64 / LPR;   // split rows per load instruction
    constexpr int U = 32;           // load instructions per lane and round
    const int lane = threadIdx.x;
    const int row = blockIdx.x;  // ((b * s_active + i) * n_q_heads + h)
    const int h = row % p.n_q_heads;
    const int i = (row / p.n_q_heads) % p.s_active;
    const int b = row / (p.n_q_heads * p.s_active);
    const int len = p.cache_len[b];
    const int ns = len > 0 ? min(p.max_splits, (len + p.split_len - 1) / p.split_len) : 0;
    const float* lse = p.part_lse + (int64_t)row * p.max_splits;
    const float* po = p.part_o + (int64_t)row * p.max_splits * D;

    const int r = lane / LPR, c = lane % LPR;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float wsum = 0.f, M = -__builtin_inff();
    for (int s0 = 0; s0 < ns; s0 += RPW * U) {
        float4 x[U];
        float ls[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int sc = min(s0 + RPW * u + r, ns - 1);  // every split below ns was written
            x[u] = *(const float4*)(po + (int64_t)sc * D + 4 * c);
            ls[u] = lse[sc];
        }
        // running max over the splits seen so far (a repeated clamped split changes nothing)
        float mr = M;
#pragma unroll
        for (int u = 0; u < U; ++u) mr = fmaxf(mr, ls[u]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mr = fmaxf(mr, __shfl_xor(mr, off));
        if (mr == -__builtin_inff()) continue;  // every split so far is empty
        const float alpha = fast_exp2((M - mr) * kLog2e);  // 0 on the first non-empty round
        M = mr;
        wsum *= alpha;
        acc.x *= alpha; acc.y *= alpha; acc.z *= alpha; acc.w *= alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float wt = s0 + RPW * u + r < ns ? fast_exp2((ls[u] - M) * kLog2e) : 0.f;
            wsum += wt;
            acc.x = fmaf(wt, x[u].x, acc.x);
            acc.y = fmaf(wt, x[u].y, acc.y);
            acc.z = fmaf(wt, x[u].z, acc.z);
            acc.w = fmaf(wt, x[u].w, acc.w);
        }
    }
    // sum over the RPW lane groups (same float4 column, different splits)
    auto add_other = [&](float v, bool sixteen) {
        const uint32_t u = __float_as_uint(v);
        auto sw = sixteen ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                          : __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    };
    if constexpr (RPW >= 2) {
        acc.x = add_other(acc.x, false); acc.y = add_other(acc.y, false);
        acc.z = add_other(acc.z, false); acc.w = add_other(acc.w, false);
        wsum = add_other(wsum, false);
    }
    if constexpr (RPW >= 4) {
        acc.x = add_other(acc.x, true); acc.y = add_other(acc.y, true);
        acc.z = add_other(acc.z, true); acc.w = add_other(acc.w, true);
        wsum = add_other(wsum, true);
    }
    // Attention sink: one more logit of the row, with no value (the decode
    // page's per-q-head sink), merged like a split with O = 0. The partial
    // LSEs are natural-log, so the sink enters in the same units.
    // A NaN or +inf sink makes the row NaN (written as NaN bits).
    float osc = 1.f;
    bool nan_row = false;
    if (p.sinks) {
        const float sk = p.sinks[h];
        nan_row = sink_gives_nan(sk);
        if (sk > -__builtin_inff() && !nan_row) {
            const float mn = fmaxf(M, sk);
            osc = fast_exp2((M - mn) * kLog2e);  // 0 when no split was visible (M = -inf)
            wsum = wsum * osc + fast_exp2((sk - mn) * kLog2e);
            M = mn;
        }
    }
    const float inv = wsum > 0.f ? osc / wsum : 0.f;
    if (p.lse && lane == 0)
        *(uint32_t*)&p.lse[row] = nan_row ? kNaN32 : __float_as_uint(wsum > 0.f ? M + __logf(wsum) : -__builtin_inff());
    if (r == 0) {
        uint16_t* orow = (uint16_t*)p.o + (int64_t)b * p.os.batch + (int64_t)i * p.os.seq + (int64_t)h * p.os.head;
        uint2 pk;
        pk.x = pack2_16<BF16>(acc.x * inv, acc.y * inv);
        pk.y = pack2_16<BF16>(acc.z * inv, acc.w * inv);
        if (nan_row) pk = make_uint2(kNaN16x2<BF16>, kNaN16x2<BF16>);
        *(uint2*)(orow + 4 * c) = pk;
    }
}

template <bool BF16, int D, int HW, int QB>
static void launch_decode_hw(const DecodeParams& p, hipStream_t s) {
    const dim3 grid((unsigned)(p.n_kv_heads / HW), (unsigned)p.max_splits, (unsigned)p.batch), block(64 * HW);
    if (!p.block_table) hipLaunchKernelGGL((decode_split<BF16, D, kDecodeFlat, HW, QB>), grid, block, 0, s, p);
    else if (p.page_shift >= 4) hipLaunchKernelGGL((decode_split<BF16, D, kDecodeFast, HW, QB>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((decode_split<BF16, D, kDecodeGeneric, HW, QB>), grid, block, 0, s, p);
}

template <bool BF16, int D, int HW, int QB>
static void launch_decode_f8_hw(const DecodeParams& p, hipStream_t s) {
    const dim3 grid((unsigned)(p.n_kv_heads / HW), (unsigned)p.max_splits, (unsigned)p.batch), block(64 * HW);
    if (!p.block_table) hipLaunchKernelGGL((decode_split_f8<BF16, D, kDecodeFlat, HW, QB>), grid, block, 0, s, p);
    else if (p.page_shift >= 4) hipLaunchKernelGGL((decode_split_f8<BF16, D, kDecodeFast, HW, QB>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((decode_split_f8<BF16, D, kDecodeGeneric, HW, QB>), grid, block, 0, s, p);
}

// Waves per workgroup: the largest power of two up to the LDS-bound maximum
// that divides n_kv_heads (decode_split_f8 holds one V tile per wave, decode_split four).
template <int D>
static int decode_heads_d(bool fp8, int n_kv_heads, int batch, int max_splits) {
    const int mh = fp8 ? dc_max_heads_f8<D>() : dc_max_heads<D>();
    const bool wide = (int64_t)batch * max_splits * (n_kv_heads / 8) >= kDecodeF8WideGrid;
    if (fp8 && mh >= 8 && n_kv_heads % 8 == 0 && wide) return 8;
    if (mh >= 4 && n_kv_heads % 4 == 0) return 4;
    if (mh >= 2 && n_kv_heads % 2 == 0) return 2;
    return 1;
}

int decode_heads_per_workgroup(bool fp8, int head_dim, int n_kv_heads, int batch, int max_splits) {
    switch (head_dim) {
        case 64: return decode_heads_d<64>(fp8, n_kv_heads, batch, max_splits);
        case 128: return decode_heads_d<128>(fp8, n_kv_heads, batch, max_splits);
        default: return decode_heads_d<256>(fp8, n_kv_heads, batch, max_splits);
    }
}

template <bool BF16, int D, int QB>
static void launch_decode_q(const DecodeParams& p, hipStream_t s) {
    const int hw = decode_heads_d<D>(p.kv_fp8, p.n_kv_heads, p.batch, p.max_splits);
    if (p.kv_fp8) {
        constexpr int MH = dc_max_heads_f8<D>();
        if (MH >= 8 && hw == 8) launch_decode_f8_hw<BF16, D, (MH >= 8 ? 8 : 1), QB>(p, s);
        else if (MH >= 4 && hw == 4) launch_decode_f8_hw<BF16, D, (MH >= 4 ? 4 : 1), QB>(p, s);
        else if (MH >= 2 && hw == 2) launch_decode_f8_hw<BF16, D, (MH >= 2 ? 2 : 1), QB>(p, s);
        else launch_decode_f8_hw<BF16, D, 1, QB>(p, s);
        return;
    }
    constexpr int MH = dc_max_heads<D>();
    if (MH >= 4 && hw == 4) launch_decode_hw<BF16, D, (MH >= 4 ? 4 : 1), QB>(p, s);
    else if (MH >= 2 && hw == 2) launch_decode_hw<BF16, D, (MH >= 2 ? 2 : 1), QB>(p, s);
    else launch_decode_hw<BF16, D, 1, QB>(p, s);
}

// More than 16 query rows per kv-head (G * s_active) take a second 16-column
// block of MFMAs over the same K/V fragments (D <= 128; the host rejects more
// than 16 rows at D = 256, whose registers leave no room for it).
template <bool BF16, int D>
static void launch_decode_d(const DecodeParams& p, hipStream_t s) {
    if constexpr (D <= 128) {
        if (p.group * p.s_active > 16) {
            launch_decode_q<BF16, D, 2>(p, s);
            return;
        }
    }
    launch_decode_q<BF16, D, 1>(p, s);
}

template <bool BF16>
static hipError_t launch_decode_t(const DecodeParams& p, int head_dim, hipStream_t s) {
    switch (head_dim) {
        case 64: launch_decode_d<BF16, 64>(p, s); break;
        case 128: launch_decode_d<BF16, 128>(p, s); break;
        default: launch_decode_d<BF16, 256>(p, s); break;
    }
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int dtype, int head_dim, hipStream_t s) {
    return dtype == kBF16 ? launch_decode_t<true>(p, head_dim, s) : launch_decode_t<false>(p, head_dim, s);
}

template <bool BF16>
static hipError_t launch_combine_t(const CombineParams& p, int head_dim, hipStream_t s) {
    const dim3 grid((unsigned)(p.batch * p.s_active * p.n_q_heads));
    switch (head_dim) {
        case 64: hipLaunchKernelGGL((decode_combine<BF16, 64>), grid, dim3(64), 0, s, p); break;
        case 128: hipLaunchKernelGGL((decode_combine<BF16, 128>), grid, dim3(64), 0, s, p); break;
        default: hipLaunchKernelGGL((decode_combine<BF16, 256>), grid, dim3(64), 0, s, p); break;
    }
    return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, int dtype, int head_dim, hipStream_t s) {
    return dtype == kBF16 ? launch_combine_t<true>(p, head_dim, s) : launch_combine_t<false>(p, head_dim, s);
}

// ---------------------------------------------------------------------------- allocation-free decode
// The split partials of attn_decode_fwd_noalloc live in this file-scope
// device array: one copy per GPU, held until the process ends, shared by
// every such call on that GPU (calls that overlap on one GPU race on it).
// Host code never uses the array's name as an address (in host code it is a
// stand-in, not device memory): its device address is looked up once per
// device, with that device current, and passed to the kernels as the
// partials' pointers, exactly as a caller's workspace would be. Nothing in it
// needs clearing: the combine reads only the splits the split kernel has just
// written (those that start below cache_len).
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_NOALLOC_MAX_BYTES];

namespace {
constexpr int kScratchMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kScratchMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** addr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_addr[dev]) {
        void* a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_addr[dev] = a;
    }
    *addr = g_scratch_addr[dev];
    return hipSuccess;
}

// Page-table validation (the device-side range check of the page indices).
// The decode page's gather faults on an out-of-range page index (section
// "Paged / block cache"), and the split kernels trust the table, so a caller
// can check it first. result[0] counts the problems, result[1] is the lowest
// flat index (b * max_pages_per_seq + page) of a bad entry, or of the first
// page slot of a sequence whose cache_len is negative or longer than its row
// of the table. Only the pages below ceil(cache_len / page_size) are checked.
__global__ __launch_bounds__(64) void validate_pages_init(int32_t* result) {
    if (threadIdx.x == 0) {
        result[0] = 0;
        result[1] = 0x7fffffff;
    }
}

__global__ __launch_bounds__(256) void validate_pages(const uint32_t* block_table, const int32_t* cache_len,
                                                      int max_pages_per_seq, int page_size, int64_t num_pages,
                                                      int32_t* result) {
    const int b = blockIdx.y;
    const int len = cache_len[b];
    const int64_t row = (int64_t)b * max_pages_per_seq;
    if (len < 0 || (int64_t)len > (int64_t)max_pages_per_seq * page_size) {
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            atomicAdd(&result[0], 1);
            atomicMin(&result[1], (int32_t)row);
        }
        return;
    }
    const int npages = (len + page_size - 1) / page_size;
    for (int i = blockIdx.x * 256 + (int)threadIdx.x; i < npages; i += gridDim.x * 256) {
        if ((int64_t)block_table[row + i] >= num_pages) {
            atomicAdd(&result[0], 1);
            atomicMin(&result[1], (int32_t)(row + i));
        }
    }
}

hipError_t launch_validate_pages(const uint32_t* block_table, const int32_t* cache_len, int batch,
                                 int max_pages_per_seq, int page_size, int64_t num_pages, int32_t* result,
                                 hipStream_t s) {
    hipLaunchKernelGGL(validate_pages_init, dim3(1), dim3(64), 0, s, result);
    if (batch > 0) {
        const unsigned gx = (unsigned)std::min(64, (max_pages_per_seq + 255) / 256);
        hipLaunchKernelGGL(validate_pages, dim3(gx, (unsigned)batch), dim3(256), 0, s, block_table, cache_len,
                           max_pages_per_seq, page_size, num_pages, result);
    }
    return hipGetLastError();
}

}  // namespace attn
