// Prefill (context) flash-attention forward for gfx950.
//
// f16 / bf16: prefill_mfma — one workgroup per (128-row Q tile, q-head,
// batch), four waves of 32 query rows each. Q stays in VGPRs as MFMA
// operands for the whole kernel ("Q resident, KV streams": CTE page,
// section "Tile shapes and residency"); 64-key K/V tiles stream through LDS,
// register-prefetched one tile ahead. Each wave computes the transposed
// score tile S^T = K Q^T with v_mfma_f32_32x32x16, so every lane owns one
// query row and the row max / row sum are in-lane plus one v_permlane32_swap.
// The f32 S^T accumulator layout is exactly the B-operand layout of
// O^T += V^T P^T, so P never leaves registers; V^T is read from the
// row-major V tile with ds_read_b64_tr_b16. O^T (f32) and m, l stay in VGPRs.
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
#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {

constexpr int PF_BM = 128;  // query rows per workgroup
constexpr int PF_BN = 64;   // keys per tile
constexpr int PF_THREADS = 256;
constexpr int PF_KPAD = 8;   // K row padding (elements): 16 B keeps 16-lane b128 reads conflict-free
constexpr int PF_VPAD = 32;  // V row padding (elements): rows land 64 B apart for the transpose reads

template <bool B>
struct BoolC {
    static constexpr bool value = B;
};

template <bool BF16, int D, int MASK>
__global__ __launch_bounds__(PF_THREADS, (D >= 256 ? 1 : 2)) void prefill_mfma(PrefillParams p) {
    constexpr int KSTR = D + PF_KPAD;
    constexpr int VSTR = D + PF_VPAD;
    constexpr int CH = PF_BN * D / 8 / PF_THREADS;  // 16-byte chunks per thread per tensor
    constexpr int NDT = D / 32;                      // 32-wide d tiles of O^T
    // Two K/V tile buffers: tile j+1 is written while tile j is read, one barrier per tile.
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][PF_BN * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][PF_BN * VSTR];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31;
    const int hf = lane >> 5;   // wave half
    const int g = lane >> 4;    // 16-lane group
    const int r16 = lane & 15;

    // Workgroup -> (q tile, batch, q-head). Consecutive workgroups are the
    // heads of one q tile; causal tiles are issued heaviest first.
    const int nbh = p.batch * p.n_q_heads;
    const int qt = p.n_q_tiles - 1 - (int)(blockIdx.x / nbh);
    const int bh = blockIdx.x % nbh;
    const int b = bh / p.n_q_heads;
    const int h = bh % p.n_q_heads;
    const int hk = h / p.group;

    const int q0 = qt * PF_BM;
    const int qlast = min(q0 + PF_BM, p.seqlen_q) - 1;
    int kv_lo = 0, kv_hi = p.seqlen_kv;
    if (MASK >= kMaskCausal) kv_hi = min(kv_hi, qlast + p.off + 1);
    if (MASK == kMaskCausalWindow) kv_lo = max(0, q0 + p.off - p.window + 1);
    const int j_begin = kv_lo / PF_BN;
    const int j_end = kv_hi > kv_lo ? (kv_hi + PF_BN - 1) / PF_BN : j_begin;

    const int wq0 = q0 + 32 * w;                   // first row of this wave
    const int wq1 = min(wq0 + 31, p.seqlen_q - 1); // last valid row of this wave
    const bool wave_live = wq0 < p.seqlen_q;
    const int my_q = wq0 + l32;                    // the query row this lane owns
    const int my_pos = my_q + p.off;

    // Q fragments: B operand of S^T = K Q^T (lane: row l32, d = 16s + 8hf .. +8).
    s16x8 qf[D / 16];
    {
        const uint16_t* qrow = (const uint16_t*)p.q + (int64_t)b * p.qs.batch + (int64_t)my_q * p.qs.seq +
                               (int64_t)h * p.qs.head + 8 * hf;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (my_q < p.seqlen_q) x = *(const uint4*)(qrow + 16 * s);
            x.x ^= p.qflip; x.y ^= p.qflip; x.z ^= p.qflip; x.w ^= p.qflip;
            qf[s] = __builtin_bit_cast(s16x8, x);
        }
    }

    const uint16_t* kbase = (const uint16_t*)p.k + (int64_t)b * p.ks.batch + (int64_t)hk * p.ks.head;
    const uint16_t* vbase = (const uint16_t*)p.v + (int64_t)b * p.vs.batch + (int64_t)hk * p.vs.head;
    uint4 kreg[CH], vreg[CH];
    auto gload = [&](int j) {
        const int kv0 = j * PF_BN;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + i * PF_THREADS;
            const int row = c / (D / 8), col = (c % (D / 8)) * 8;
            const int key = kv0 + row;
            kreg[i] = make_uint4(0, 0, 0, 0);
            vreg[i] = make_uint4(0, 0, 0, 0);
            // rows outside [kv_lo, seqlen_kv) are never visible to this tile: zero them
            if (key < p.seqlen_kv && key >= kv_lo) {
                kreg[i] = *(const uint4*)(kbase + (int64_t)key * p.ks.seq + col);
                vreg[i] = *(const uint4*)(vbase + (int64_t)key * p.vs.seq + col);
            }
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + i * PF_THREADS;
            const int row = c / (D / 8), col = (c % (D / 8)) * 8;
            *(uint4*)&Ks[buf][row * KSTR + col] = kreg[i];
            *(uint4*)&Vs[buf][row * VSTR + col] = vreg[i];
        }
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

    auto tile = [&](const uint16_t* Kt, const uint16_t* Vt, int kv0, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        // S^T tile: two 32-key blocks x 32 queries; lane holds keys
        // 32t + 8(r/4) + 4hf + r%4 of its query row in register r.
        f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const s16x8 a = *(const s16x8*)&Kt[(32 * t + l32) * KSTR + 16 * s + 8 * hf];
                sacc[t] = mfma32x32x16<BF16>(a, qf[s], sacc[t]);
            }
        }
        if constexpr (!FULL) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + 32 * t + 8 * (r >> 2) + 4 * hf + (r & 3);
                    bool keep = key < p.seqlen_kv;
                    if (MASK >= kMaskCausal) keep &= key <= my_pos;
                    if (MASK == kMaskCausalWindow) keep &= key >= my_pos - p.window + 1;
                    sacc[t][r] = keep ? sacc[t][r] : kMaskedScore;
                }
        }
        float mx = kMaskedScore;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[t][r]);
        mx = max_with_other_half(mx);
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

        // P in 16-bit, packed as the B operand of O^T += V^T P^T: chunk u
        // covers keys 16u..16u+15 of the tile; slot j of lane half hf is key
        // 16u + 8(j/4) + 4hf + j%4, i.e. register 8(u%2) + j of block u/2.
        s16x8 pb[4];
        float psum = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint32_t pk[4];
#pragma unroll
            for (int jj = 0; jj < 8; jj += 2) {
                const float s0 = sacc[u >> 1][8 * (u & 1) + jj];
                const float s1 = sacc[u >> 1][8 * (u & 1) + jj + 1];
                float p0 = fast_exp2(fmaf(s0, p.c, neg_m));
                float p1 = fast_exp2(fmaf(s1, p.c, neg_m));
                if constexpr (!FULL) {
                    p0 = s0 == kMaskedScore ? 0.f : p0;
                    p1 = s1 == kMaskedScore ? 0.f : p1;
                }
                pk[jj / 2] = pack2_16<BF16>(p0, p1);
                psum = dot2_16<BF16>(pk[jj / 2], one2, psum);  // sum of the rounded P
            }
            pb[u] = __builtin_bit_cast(s16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
        }
        l_i += psum;

        // O^T[d, q] += V^T[d, keys] P^T[keys, q]. A operand via transpose
        // reads: lane r16 of group g points at row 16u + 4hf + r16/4 (and +8),
        // column 32dt + 16(g%2) + 4(r16%4), and receives column 32dt + 16(g%2)
        // + r16 of four consecutive key rows.
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int row0 = 16 * u + 4 * hf + (r16 >> 2);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const int col = 32 * dt + 16 * (g & 1) + 4 * (r16 & 3);
                const s16x4 lo = lds_read_tr16(&Vt[row0 * VSTR + col]);
                const s16x4 hi4 = lds_read_tr16(&Vt[(row0 + 8) * VSTR + col]);
                o[dt] = mfma32x32x16<BF16>(concat4(lo, hi4), pb[u], o[dt]);
            }
        }
    };

    if (j_begin < j_end) {
        gload(j_begin);
        lstore(0);
        __syncthreads();
        if (j_begin + 1 < j_end) gload(j_begin + 1);
    }
    for (int j = j_begin; j < j_end; ++j) {
        const int buf = (j - j_begin) & 1;
        const int kv0 = j * PF_BN;
        bool empty = !wave_live;
        if (MASK >= kMaskCausal) empty |= kv0 > wq1 + p.off;
        if (MASK == kMaskCausalWindow) empty |= kv0 + PF_BN - 1 < wq0 + p.off - p.window + 1;
        if (!empty) {
            bool full = kv0 + PF_BN <= p.seqlen_kv;
            if (MASK >= kMaskCausal) full &= kv0 + PF_BN - 1 <= wq0 + p.off;
            if (MASK == kMaskCausalWindow) full &= kv0 >= wq1 + p.off - p.window + 1;
            if (full) tile(Ks[buf], Vs[buf], kv0, BoolC<true>{});
            else tile(Ks[buf], Vs[buf], kv0, BoolC<false>{});
        }
        if (j + 1 < j_end) lstore(buf ^ 1);  // the other buffer's tile (j-1) is done: barrier of the last step
        __syncthreads();
        if (j + 2 < j_end) gload(j + 2);
    }

    // Epilogue: O * (1/l); rows that saw no key are written as zeros.
    const float l_tot = sum_with_other_half(l_i);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (wave_live && my_q < p.seqlen_q) {
        uint16_t* orow = (uint16_t*)p.o + (int64_t)b * p.os.batch + (int64_t)my_q * p.os.seq +
                         (int64_t)h * p.os.head;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int d = 32 * dt + 8 * rq + 4 * hf;
                uint2 pk;
                pk.x = pack2_16<BF16>(o[dt][4 * rq + 0] * inv, o[dt][4 * rq + 1] * inv);
                pk.y = pack2_16<BF16>(o[dt][4 * rq + 2] * inv, o[dt][4 * rq + 3] * inv);
                *(uint2*)(orow + d) = pk;
            }
    }
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
    const int q0 = qt * F32_BM;
    const int qlast = min(q0 + F32_BM, p.seqlen_q) - 1;
    int kv_lo = 0, kv_hi = p.seqlen_kv;
    if (MASK >= kMaskCausal) kv_hi = min(kv_hi, qlast + p.off + 1);
    if (MASK == kMaskCausalWindow) kv_lo = max(0, q0 + p.off - p.window + 1);
    const int j_begin = kv_lo / F32_BN;
    const int j_end = kv_hi > kv_lo ? (kv_hi + F32_BN - 1) / F32_BN : j_begin;

    const int my_q = q0 + r, my_pos = my_q + p.off;
    const bool live = my_q < p.seqlen_q;
    float qv[DQ], acc[DQ];
    {
        const float* qrow = (const float*)p.q + (int64_t)b * p.qs.batch + (int64_t)my_q * p.qs.seq +
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
    const float* kbase = (const float*)p.k + (int64_t)b * p.ks.batch + (int64_t)hk * p.ks.head;
    const float* vbase = (const float*)p.v + (int64_t)b * p.vs.batch + (int64_t)hk * p.vs.head;
    float m_i = kMaxInit, l_i = 0.f;

    for (int j = j_begin; j < j_end; ++j) {
        const int kv0 = j * F32_BN;
        __syncthreads();
        for (int c = tid; c < F32_BN * D / 4; c += 256) {
            const int row = c / (D / 4), col = (c % (D / 4)) * 4;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (kv0 + row < p.seqlen_kv && kv0 + row >= kv_lo) {
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
            bool keep = key < p.seqlen_kv;
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
        const float inv = l_i > 0.f ? 1.f / l_i : 0.f;
        float* orow = (float*)p.o + (int64_t)b * p.os.batch + (int64_t)my_q * p.os.seq + (int64_t)h * p.os.head +
                      qd * DQ;
#pragma unroll
        for (int e = 0; e < DQ; e += 4)
            *(float4*)(orow + e) = make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
    }
}

// ---------------------------------------------------------------------------- dispatch
template <bool BF16, int D>
static hipError_t launch_mfma_mask(PrefillParams p, int mask, hipStream_t s) {
    p.n_q_tiles = (p.seqlen_q + PF_BM - 1) / PF_BM;
    const dim3 grid((unsigned)p.n_q_tiles * p.batch * p.n_q_heads);
    switch (mask) {
        case kMaskNone: hipLaunchKernelGGL((prefill_mfma<BF16, D, kMaskNone>), grid, dim3(PF_THREADS), 0, s, p); break;
        case kMaskCausal: hipLaunchKernelGGL((prefill_mfma<BF16, D, kMaskCausal>), grid, dim3(PF_THREADS), 0, s, p); break;
        default: hipLaunchKernelGGL((prefill_mfma<BF16, D, kMaskCausalWindow>), grid, dim3(PF_THREADS), 0, s, p); break;
    }
    return hipGetLastError();
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

template <bool BF16>
static hipError_t launch_mfma_d(const PrefillParams& p, int head_dim, int mask, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_mfma_mask<BF16, 64>(p, mask, s);
        case 128: return launch_mfma_mask<BF16, 128>(p, mask, s);
        default: return launch_mfma_mask<BF16, 256>(p, mask, s);
    }
}

hipError_t launch_prefill(const PrefillParams& p, int dtype, int head_dim, int mask, hipStream_t s) {
    if (dtype == kF32) {
        switch (head_dim) {
            case 64: return launch_f32_mask<64>(p, mask, s);
            case 128: return launch_f32_mask<128>(p, mask, s);
            default: return launch_f32_mask<256>(p, mask, s);
        }
    }
    return dtype == kBF16 ? launch_mfma_d<true>(p, head_dim, mask, s) : launch_mfma_d<false>(p, head_dim, mask, s);
}

}  // namespace attn
