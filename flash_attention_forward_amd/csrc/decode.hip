// Split-KV decode attention and the log-sum-exp combine for gfx950.
//
// decode_split: one wavefront per (split, kv-head, sequence). The G * s_active
// query rows that share a kv-head (G = n_q_heads / n_kv_heads) ride one MFMA
// together, so each K/V byte is read once for all of them — the decode page's
// grouped-query "free broadcast" ("Flash-Attention: Decode (TKG)", section
// "GQA / MQA grouped-query broadcast"), done here with v_mfma_f32_16x16x32
// (16 key rows x 16 query columns, query columns beyond G * s_active are
// zero). Keys are gathered through the uint32 page table, 32 per iteration
// (decode page, section "Paged / block cache"): K goes from HBM straight into
// the MFMA A operand, V is staged through LDS and read back transposed with
// ds_read_b64_tr_b16 for O^T += V^T P^T. The next 32 keys are in flight while
// the current ones are used. Rows of a split's last page at or beyond
// cache_len are neither read nor used (decode page, section "gen_mask_tkg":
// index < cache length), and their V rows are zero so that nothing there can
// leak into the product.
//
// Each split writes its normalised output and its natural-log log-sum-exp
// (the decode page's deferred normalisation on its flash path: the partial
// output plus the statistics needed to merge it later).
//
// decode_combine: per (sequence, query, q-head), M = max_s lse_s,
// w_s = exp(lse_s - M), O = sum_s w_s O_s / sum_s w_s — the CTE page's
// cross-section merge (section "Algorithm — running-sum update, reciprocal,
// output accumulate") over any number of splits.
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

template <bool BF16, int D, int MODE>
__global__ __launch_bounds__(64, (D >= 256 ? 1 : 2)) void decode_split(DecodeParams p) {
    constexpr int NKS = D / 32;              // k-steps of S^T = K Q^T
    constexpr int NDT = D / 16;              // 16-row d tiles of O^T
    constexpr int CPR = D / 8;               // 16-byte chunks per V row
    constexpr int RPL = 64 / CPR;            // V rows covered by one direct-to-LDS load
    constexpr int VLD = DC_KB / RPL;         // direct-to-LDS loads per lane per block
    constexpr int KLD = 2 * NKS;             // K loads per lane per block
    // Two V tiles in LDS and two K register sets: block i+2 is requested while
    // block i is used, so each block's loads have a whole iteration to land.
    __shared__ __attribute__((aligned(16))) uint16_t VsA[DC_KB * D];
    __shared__ __attribute__((aligned(16))) uint16_t VsB[DC_KB * D];
    // This split's slice of the page table, read once: address generation in
    // the loop then never waits on a global load.
    __shared__ uint32_t pages[kDecodeMaxSplitPages];

    const int lane = threadIdx.x;
    const int n = lane & 15;   // query column / key row within a 16-block
    const int g = lane >> 4;   // 16-lane group
    // x = kv-head fastest: the waves of one split are dispatched together and
    // read the same pages at about the same time.
    const int hk = blockIdx.x, split = blockIdx.y, b = blockIdx.z;

    const int len = p.cache_len[b];
    const int t0 = split * p.split_len;
    if (t0 >= len) return;  // this split is past the cache: nothing is written
    const int t1 = min(len, t0 + p.split_len);

    const int nrows = p.group * p.s_active;
    const bool row_real = n < nrows;
    const int qi = row_real ? n / p.group : 0;
    const int qh = hk * p.group + (row_real ? n % p.group : 0);
    const int qpos = len - p.s_active + qi;  // the query sits at the end of its cache
    const int64_t prow = (((int64_t)b * p.s_active + qi) * p.n_q_heads + qh) * p.max_splits + split;

    // Keys this split may use: [t0, t1) clipped to the window of the earliest query.
    int tlo = t0;
    if (p.window > 0) tlo = max(tlo, (len - p.s_active) - p.window + 1);
    if (tlo >= t1) {  // no visible key: empty partial
        if (row_real) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                *(float4*)(p.part_o + prow * D + 16 * dt + 4 * g) = make_float4(0.f, 0.f, 0.f, 0.f);
            if (g == 0) p.part_lse[prow] = -__builtin_inff();
        }
        return;
    }
    const int tb0 = t0 + ((tlo - t0) / DC_KB) * DC_KB;  // first iteration's key block
    const int nblk = (t1 - tb0 + DC_KB - 1) / DC_KB;
    if constexpr (MODE != kDecodeFlat) {
        // pages holding tokens [t0, t1); t0 is a multiple of page_size
        const int first = t0 / p.page_size;
        const int npg = (t1 - 1) / p.page_size - first + 1;
        const uint32_t* row = p.block_table + (int64_t)b * p.max_pages_per_seq + first;
        for (int i = lane; i < npg; i += 64) pages[i] = row[i];
        __syncthreads();
    }

    // Q fragments: B operand of S^T = K Q^T (lane: column n, d = 32ks + 8g .. +8).
    s16x8 qf[NKS];
    {
        const uint16_t* qrow = (const uint16_t*)p.q + (int64_t)b * p.qs.batch + (int64_t)qi * p.qs.seq +
                               (int64_t)qh * p.qs.head + 8 * g;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (row_real) x = *(const uint4*)(qrow + 32 * ks);
            x.x ^= p.qflip; x.y ^= p.qflip; x.z ^= p.qflip; x.w ^= p.qflip;
            qf[ks] = __builtin_bit_cast(s16x8, x);
        }
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
    // token: rows past the end (and whole blocks past the last one) re-read
    // finite cache data, get probability exactly 0 in the softmax and so add
    // exactly nothing to P V. Nothing at or beyond cache_len is ever read. With
    // no conditional loads, each lane has exactly KLD + VLD loads per block in
    // flight and the wait counts below hold on every path.
    const int tlast = t1 - 1;
    // FAST: offset of the 16-aligned group holding token t, plus the row within it
    auto fast_off = [&](int t) -> int64_t {
        const int tc = min(t, tlast);
        const int tg = tc & ~15;
        return row_off(tg) + (int64_t)(tc - tg) * seq;
    };
    auto load_k = [&](uint4 (&kr)[2][NKS], int tb) {
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
            const int t = tb + 16 * gi + n;
            const uint16_t* src = kbase + (MODE == kDecodeGeneric ? row_off(min(t, tlast)) : fast_off(t)) + 8 * g;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) kr[gi][ks] = *(const uint4*)(src + 32 * ks);
        }
    };
    // V block straight into LDS: load i writes LDS bytes [1 KB * i, 1 KB * (i + 1)),
    // lane L landing at row i * RPL + L / CPR, swizzled chunk L % CPR.
    const int cs = lane % CPR;
    auto load_v = [&](uint16_t* V, int tb) {
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int row = i * RPL + lane / CPR;
            const int t = tb + row;
            const int c = cs ^ dc_vswz<D>(row);
            const int64_t off = MODE == kDecodeGeneric ? row_off(min(t, tlast)) : fast_off(t);
            __builtin_amdgcn_global_load_lds(vbase + off + 8 * c, (__attribute__((address_space(3))) void*)(V + 512 * i),
                                             16, 0, 0);
        }
    };
    float m_i = kMaxInit, l_i = 0.f;
    f32x4 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{};
    const uint32_t one2 = BF16 ? 0x3F803F80u : 0x3C003C00u;

    // One block: wait for its loads, S^T = K Q^T, refill these K registers with
    // block it+2, online softmax, O^T += V^T P^T, refill this V tile with block it+2.
    auto step = [&](uint4 (&kr)[2][NKS], uint16_t* V, int it) {
        const int tb = tb0 + it * DC_KB;
        wait_vmcnt<KLD + VLD>();  // only block it+1's loads may still be in flight
        __syncthreads();

        f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int gi = 0; gi < 2; ++gi)
                sacc[gi] = mfma16x16x32<BF16>(__builtin_bit_cast(s16x8, kr[gi][ks]), qf[ks], sacc[gi]);
        load_k(kr, tb + 2 * DC_KB);  // block it+2 (clamped rows when past the end)

        // rows at or beyond t1 hold another row's keys: masked here
        float mx = kMaskedScore;
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = tb + 16 * gi + 4 * g + r;
                bool keep = t < t1 && t <= qpos;
                if (p.window > 0) keep &= t >= qpos - p.window + 1;
                sacc[gi][r] = keep ? sacc[gi][r] : kMaskedScore;
                mx = fmaxf(mx, sacc[gi][r]);
            }
        mx = max_over_groups(mx);
        const float m_new = fmaxf(m_i, mx * p.c);
        const float alpha = fast_exp2(m_i - m_new);
        m_i = m_new;

        // P^T as the B operand: slot j of group g is key 4g + j (j < 4) or 16 + 4g + j - 4.
        uint32_t pk[4];
        float psum = 0.f;
#pragma unroll
        for (int jj = 0; jj < 8; jj += 2) {
            const float s0 = sacc[jj >> 2][jj & 3], s1 = sacc[jj >> 2][(jj & 3) + 1];
            const float p0 = s0 == kMaskedScore ? 0.f : fast_exp2(fmaf(s0, p.c, -m_new));
            const float p1 = s1 == kMaskedScore ? 0.f : fast_exp2(fmaf(s1, p.c, -m_new));
            pk[jj / 2] = pack2_16<BF16>(p0, p1);
            psum = dot2_16<BF16>(pk[jj / 2], one2, psum);
        }
        const s16x8 pb = __builtin_bit_cast(s16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
        l_i = l_i * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;

        // O^T[d, q] += V^T[d, keys] P^T[keys, q]; lane n of group g reads rows
        // 4g + n/4 (and 16 + ...), column 16dt + 4(n%4), receiving column 16dt + n.
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int c = 2 * dt + ((n & 3) >> 1), half = 4 * (n & 1);
            const int r0 = 4 * g + (n >> 2), r1 = r0 + 16;
            const s16x4 lo = lds_read_tr16(&V[r0 * D + 8 * (c ^ dc_vswz<D>(r0)) + half]);
            const s16x4 hi4 = lds_read_tr16(&V[r1 * D + 8 * (c ^ dc_vswz<D>(r1)) + half]);
            o[dt] = mfma16x16x32<BF16>(concat4(lo, hi4), pb, o[dt]);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // transpose reads done before the tile is refilled
        __syncthreads();
        load_v(V, tb + 2 * DC_KB);
    };

    uint4 ka[2][NKS], kb[2][NKS];
    load_k(ka, tb0);
    load_v(VsA, tb0);
    load_k(kb, tb0 + DC_KB);
    load_v(VsB, tb0 + DC_KB);
    // An odd block count runs one extra, fully masked block (no loads beyond the clamp).
    for (int it = 0; it < nblk; it += 2) {
        step(ka, VsA, it);
        step(kb, VsB, it + 1);
    }
    wait_vmcnt<0>();  // drain the clamped prefetches before the wave ends

    const float l_tot = sum_over_groups(l_i);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (row_real) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            *(float4*)(p.part_o + prow * D + 16 * dt + 4 * g) =
                make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
        if (g == 0) p.part_lse[prow] = l_tot > 0.f ? (m_i + __log2f(l_tot)) * 0.69314718055994531f : -__builtin_inff();
    }
}

template <bool BF16, int D>
__global__ __launch_bounds__(64) void decode_combine(CombineParams p) {
    constexpr int PER = D / 64;
    constexpr int MAXS = 256;  // splits weighted in parallel per pass
    __shared__ float wts[MAXS];
    const int lane = threadIdx.x;
    const int row = blockIdx.x;  // ((b * s_active + i) * n_q_heads + h)
    const int h = row % p.n_q_heads;
    const int i = (row / p.n_q_heads) % p.s_active;
    const int b = row / (p.n_q_heads * p.s_active);
    const int len = p.cache_len[b];
    const int ns = len > 0 ? min(p.max_splits, (len + p.split_len - 1) / p.split_len) : 0;
    const float* lse = p.part_lse + (int64_t)row * p.max_splits;
    const float* po = p.part_o + (int64_t)row * p.max_splits * D;

    // M = max_s lse_s, one split per lane, then a wave reduction
    float M = -__builtin_inff();
    for (int s = lane; s < ns; s += 64) M = fmaxf(M, lse[s]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));

    float acc[PER], wsum = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    if (M > -__builtin_inff()) {
        for (int s0 = 0; s0 < ns; s0 += MAXS) {
            const int cnt = min(MAXS, ns - s0);
            __syncthreads();
            for (int s = lane; s < cnt; s += 64) wts[s] = fast_exp2((lse[s0 + s] - M) * kLog2e);
            __syncthreads();
            int s = 0;
            for (; s + 4 <= cnt; s += 4) {  // four independent loads in flight per lane
                float x[4][PER];
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int e = 0; e < PER; ++e) x[u][e] = po[(int64_t)(s0 + s + u) * D + lane + 64 * e];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    wsum += wts[s + u];
#pragma unroll
                    for (int e = 0; e < PER; ++e) acc[e] = fmaf(wts[s + u], x[u][e], acc[e]);
                }
            }
            for (; s < cnt; ++s) {
                wsum += wts[s];
#pragma unroll
                for (int e = 0; e < PER; ++e) acc[e] = fmaf(wts[s], po[(int64_t)(s0 + s) * D + lane + 64 * e], acc[e]);
            }
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    uint16_t* orow = (uint16_t*)p.o + (int64_t)b * p.os.batch + (int64_t)i * p.os.seq + (int64_t)h * p.os.head;
#pragma unroll
    for (int e = 0; e < PER; ++e) orow[lane + 64 * e] = f32_to_16<BF16>(acc[e] * inv);
}

template <bool BF16, int D>
static void launch_decode_d(const DecodeParams& p, dim3 grid, hipStream_t s) {
    if (!p.block_table) hipLaunchKernelGGL((decode_split<BF16, D, kDecodeFlat>), grid, dim3(64), 0, s, p);
    else if (p.page_shift >= 4) hipLaunchKernelGGL((decode_split<BF16, D, kDecodeFast>), grid, dim3(64), 0, s, p);
    else hipLaunchKernelGGL((decode_split<BF16, D, kDecodeGeneric>), grid, dim3(64), 0, s, p);
}

template <bool BF16>
static hipError_t launch_decode_t(const DecodeParams& p, int head_dim, hipStream_t s) {
    const dim3 grid((unsigned)p.n_kv_heads, (unsigned)p.max_splits, (unsigned)p.batch);
    switch (head_dim) {
        case 64: launch_decode_d<BF16, 64>(p, grid, s); break;
        case 128: launch_decode_d<BF16, 128>(p, grid, s); break;
        default: launch_decode_d<BF16, 256>(p, grid, s); break;
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

}  // namespace attn
