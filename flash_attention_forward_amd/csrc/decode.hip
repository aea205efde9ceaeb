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
constexpr int DC_VPAD = 16; // V row padding (elements): transpose reads of 8 rows hit distinct banks

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

template <bool BF16, int D>
__global__ __launch_bounds__(64) void decode_split(DecodeParams p) {
    constexpr int NKS = D / 32;    // k-steps of S^T = K Q^T
    constexpr int NDT = D / 16;    // 16-row d tiles of O^T
    constexpr int VSTR = D + DC_VPAD;
    constexpr int VCH = DC_KB * D / 8 / 64;  // 16-byte V chunks per lane per iteration
    __shared__ __attribute__((aligned(16))) uint16_t Vs[DC_KB * VSTR];

    const int lane = threadIdx.x;
    const int n = lane & 15;   // query column / key row within a 16-block
    const int g = lane >> 4;   // 16-lane group
    const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;

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

    const uint16_t* kbase = (const uint16_t*)p.k + (int64_t)hk * p.kvs.head;
    const uint16_t* vbase = (const uint16_t*)p.v + (int64_t)hk * p.kvs.head;
    // Element offset of token t's row (paged: through the page table).
    auto row_off = [&](int t) -> int64_t {
        if (p.block_table) {
            const uint32_t page = p.block_table[(int64_t)b * p.max_pages_per_seq + t / p.page_size];
            return (int64_t)page * p.kvs.batch + (int64_t)(t % p.page_size) * p.kvs.seq;
        }
        return (int64_t)b * p.kvs.batch + (int64_t)t * p.kvs.seq;
    };

    uint4 kcur[2][NKS], knext[2][NKS], vreg[VCH];
    auto load_k = [&](uint4 (&kr)[2][NKS], int tb) {
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
            const int t = tb + 16 * gi + n;
            const bool ok = t < t1;
            const uint16_t* src = kbase + (ok ? row_off(t) : 0) + 8 * g;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) kr[gi][ks] = ok ? *(const uint4*)(src + 32 * ks) : make_uint4(0, 0, 0, 0);
        }
    };
    auto load_v = [&](int tb) {
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int c = lane + 64 * i;
            const int row = c / (D / 8), col = (c % (D / 8)) * 8;
            const int t = tb + row;
            vreg[i] = t < t1 ? *(const uint4*)(vbase + row_off(t) + col) : make_uint4(0, 0, 0, 0);
        }
    };

    float m_i = kMaxInit, l_i = 0.f;
    f32x4 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{};

    load_k(kcur, tb0);
    load_v(tb0);
    for (int it = 0; it < nblk; ++it) {
        const int tb = tb0 + it * DC_KB;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int c = lane + 64 * i;
            const int row = c / (D / 8), col = (c % (D / 8)) * 8;
            *(uint4*)&Vs[row * VSTR + col] = vreg[i];
        }
        __syncthreads();
        if (it + 1 < nblk) {
            load_k(knext, tb + DC_KB);
            load_v(tb + DC_KB);
        }

        // S^T: lane (n, g) holds keys tb + 16gi + 4g + r of query column n.
        f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int gi = 0; gi < 2; ++gi)
                sacc[gi] = mfma16x16x32<BF16>(__builtin_bit_cast(s16x8, kcur[gi][ks]), qf[ks], sacc[gi]);

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
        s16x8 pb;
        float psum = 0.f;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const float s = sacc[jj >> 2][jj & 3];
            const float pv = s == kMaskedScore ? 0.f : fast_exp2(fmaf(s, p.c, -m_new));
            const uint16_t pr = f32_to_16<BF16>(pv);
            psum += f16bits_to_f32<BF16>(pr);
            pb[jj] = (short)pr;
        }
        l_i = l_i * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;

        // O^T[d, q] += V^T[d, keys] P^T[keys, q]; lane n of group g reads rows
        // 4g + n/4 (and 16 + ...), column 16dt + 4(n%4), receiving column 16dt + n.
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int col = 16 * dt + 4 * (n & 3);
            const int row0 = 4 * g + (n >> 2);
            const s16x4 lo = lds_read_tr16(&Vs[row0 * VSTR + col]);
            const s16x4 hi4 = lds_read_tr16(&Vs[(row0 + 16) * VSTR + col]);
            o[dt] = mfma16x16x32<BF16>(concat4(lo, hi4), pb, o[dt]);
        }

#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) kcur[gi][ks] = knext[gi][ks];
    }

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
    const int lane = threadIdx.x;
    const int row = blockIdx.x;  // ((b * s_active + i) * n_q_heads + h)
    const int h = row % p.n_q_heads;
    const int i = (row / p.n_q_heads) % p.s_active;
    const int b = row / (p.n_q_heads * p.s_active);
    const int len = p.cache_len[b];
    const int ns = len > 0 ? min(p.max_splits, (len + p.split_len - 1) / p.split_len) : 0;
    const float* lse = p.part_lse + (int64_t)row * p.max_splits;
    const float* po = p.part_o + (int64_t)row * p.max_splits * D;

    float M = -__builtin_inff();
    for (int s = 0; s < ns; ++s) M = fmaxf(M, lse[s]);
    float acc[PER], wsum = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    if (M > -__builtin_inff()) {
        for (int s = 0; s < ns; ++s) {
            const float wgt = fast_exp2((lse[s] - M) * kLog2e);
            wsum += wgt;
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] = fmaf(wgt, po[(int64_t)s * D + lane + 64 * e], acc[e]);
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    uint16_t* orow = (uint16_t*)p.o + (int64_t)b * p.os.batch + (int64_t)i * p.os.seq + (int64_t)h * p.os.head;
#pragma unroll
    for (int e = 0; e < PER; ++e) orow[lane + 64 * e] = f32_to_16<BF16>(acc[e] * inv);
}

template <bool BF16>
static hipError_t launch_decode_t(const DecodeParams& p, int head_dim, hipStream_t s) {
    const dim3 grid((unsigned)p.max_splits, (unsigned)p.n_kv_heads, (unsigned)p.batch);
    switch (head_dim) {
        case 64: hipLaunchKernelGGL((decode_split<BF16, 64>), grid, dim3(64), 0, s, p); break;
        case 128: hipLaunchKernelGGL((decode_split<BF16, 128>), grid, dim3(64), 0, s, p); break;
        default: hipLaunchKernelGGL((decode_split<BF16, 256>), grid, dim3(64), 0, s, p); break;
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
