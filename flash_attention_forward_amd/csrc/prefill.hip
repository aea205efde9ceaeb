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

template <bool B>
struct BoolC {
    static constexpr bool value = B;
};

constexpr int PF_BM = 128;  // query rows per workgroup
constexpr int PF_BN = 64;   // keys per tile
constexpr int PF_THREADS = 256;

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

template <bool BF16, int D, int MASK>
__global__ __launch_bounds__(PF_THREADS, (D >= 256 ? 1 : 2)) void prefill_mfma(PrefillParams p) {
    constexpr int CPR = D / 8;              // 16-byte chunks per row
    constexpr int TILE = PF_BN * D;         // elements of one K or V tile
    constexpr int LPW = TILE / 512 / 4;     // 1 KB direct loads per wave per tile
    constexpr int NDT = D / 32;             // 32-wide d tiles of O^T
    // Two K and two V tiles, separate objects so waits on one buffer's refill
    // never cover reads of the other.
    __shared__ __attribute__((aligned(16))) uint16_t Ks0[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Ks1[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vs0[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vs1[TILE];

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
    // Tile rows outside [kv_lo, seqlen_kv) are loaded as copies of the nearest
    // valid row: they are masked out (probability exactly 0) and no memory
    // outside the visible key range is touched. Every load is unconditional.
    const int key_min = kv_lo, key_max = p.seqlen_kv - 1;
    // Lane part of each direct load's source offset (row within the tile and
    // swizzled chunk), computed once: interior tiles then only add a uniform
    // tile base. Edge tiles clamp row by row.
    int koff[LPW], voff[LPW];
#pragma unroll
    for (int ii = 0; ii < LPW; ++ii) {
        const int slot = 64 * (w * LPW + ii) + lane;
        const int row = slot / CPR, cs = slot % CPR;
        koff[ii] = row * (int)p.ks.seq + 8 * (cs ^ pf_kswz<D>(row));
        voff[ii] = row * (int)p.vs.seq + 8 * (cs ^ pf_vswz<D>(row));
    }
    // (Two plain lambdas rather than one generic one: a generic lambda that
    // captures these arrays keeps the compiler's host pass from emitting the
    // kernel's launch stub.)
    auto load_tile_impl = [&](uint16_t* dst, const uint16_t* base, int64_t seq, int j, const int* off, bool is_k) {
        const int kv0 = j * PF_BN;
        if (kv0 >= key_min && kv0 + PF_BN - 1 <= key_max) {
            const uint16_t* tbase = base + (int64_t)kv0 * seq;
#pragma unroll
            for (int ii = 0; ii < LPW; ++ii)
                __builtin_amdgcn_global_load_lds(tbase + off[ii],
                                                 (__attribute__((address_space(3))) void*)(dst + 512 * (w * LPW + ii)),
                                                 16, 0, 0);
        } else {
#pragma unroll
            for (int ii = 0; ii < LPW; ++ii) {
                const int i = w * LPW + ii;
                const int slot = 64 * i + lane;
                const int row = slot / CPR, cs = slot % CPR;
                const int key = min(max(kv0 + row, key_min), key_max);
                const int c = cs ^ (is_k ? pf_kswz<D>(row) : pf_vswz<D>(row));
                __builtin_amdgcn_global_load_lds(base + (int64_t)key * seq + 8 * c,
                                                 (__attribute__((address_space(3))) void*)(dst + 512 * i), 16, 0, 0);
            }
        }
    };
    auto load_k_tile = [&](uint16_t* dst, int j) { load_tile_impl(dst, kbase, p.ks.seq, j, koff, true); };
    auto load_v_tile = [&](uint16_t* dst, int j) { load_tile_impl(dst, vbase, p.vs.seq, j, voff, false); };

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

    auto tile_empty = [&](int j) {
        const int kv0 = j * PF_BN;
        bool e = !wave_live || j >= j_end;
        if (MASK >= kMaskCausal) e |= kv0 > wq1 + p.off;
        if (MASK == kMaskCausalWindow) e |= kv0 + PF_BN - 1 < wq0 + p.off - p.window + 1;
        return e;
    };
    auto tile_full = [&](int j) {
        const int kv0 = j * PF_BN;
        bool f = kv0 + PF_BN <= p.seqlen_kv;
        if (MASK >= kMaskCausal) f &= kv0 + PF_BN - 1 <= wq0 + p.off;
        if (MASK == kMaskCausalWindow) f &= kv0 >= wq1 + p.off - p.window + 1;
        return f;
    };

    // S^T: two 32-key blocks x 32 queries; lane holds keys
    // 32t + 8(r/4) + 4hf + r%4 of its query row in register r of block t.
    auto qk_half = [&](f32x16& sacc, const uint16_t* Kt, int t) {
        sacc = f32x16{};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const int row = 32 * t + l32;
            const s16x8 a = *(const s16x8*)&Kt[row * D + 8 * ((2 * s + hf) ^ pf_kswz<D>(row))];
            sacc = mfma32x32x16<BF16>(a, qf[s], sacc);
        }
    };
    auto mask_half = [&](f32x16& sacc, int kv0, int t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * t + 8 * (r >> 2) + 4 * hf + (r & 3);
            bool keep = key < p.seqlen_kv;
            if (MASK >= kMaskCausal) keep &= key <= my_pos;
            if (MASK == kMaskCausalWindow) keep &= key >= my_pos - p.window + 1;
            sacc[r] = keep ? sacc[r] : kMaskedScore;
        }
    };
    auto max_half = [&](const f32x16& sacc) {
        float mx = kMaskedScore;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
        return mx;
    };
    // P for one 32-key block, packed as B operands of O^T += V^T P^T: chunk
    // u (keys 16u..16u+15) takes registers 8(u%2)..8(u%2)+7 of block u/2; slot
    // j of lane half hf is key 16u + 8(j/4) + 4hf + j%4. Masked scores
    // (float32 min) give exactly 0: the host keeps p.c >= 1e-30.
    auto softmax_half = [&](const f32x16& sacc, s16x8& pb0, s16x8& pb1) {
        const float neg_m = -m_i;
        float psum = 0.f;
        uint32_t pk[8];
#pragma unroll
        for (int jj = 0; jj < 16; jj += 2) {
            const float p0 = fast_exp2(fmaf(sacc[jj], p.c, neg_m));
            const float p1 = fast_exp2(fmaf(sacc[jj + 1], p.c, neg_m));
            pk[jj / 2] = pack2_16<BF16>(p0, p1);
            psum = dot2_16<BF16>(pk[jj / 2], one2, psum);  // sum of the rounded P
        }
        pb0 = __builtin_bit_cast(s16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
        pb1 = __builtin_bit_cast(s16x8, make_uint4(pk[4], pk[5], pk[6], pk[7]));
        return psum;
    };
    // O^T[d, q] += V^T[d, keys] P^T[keys, q] for key chunk u. A operand via
    // transpose reads: lane r16 of group g points at row 16u + 4hf + r16/4
    // (and +8), column 32dt + 16(g%2) + 4(r16%4), and receives column
    // 32dt + 16(g%2) + r16 of four consecutive key rows.
    auto pv_chunk = [&](const s16x8& pb, const uint16_t* Vt, int u) {
        const int r0 = 16 * u + 4 * hf + (r16 >> 2), r1 = r0 + 8;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int c = 4 * dt + 2 * (g & 1) + ((r16 & 3) >> 1), e = 4 * (r16 & 1);
            const s16x4 lo = lds_read_tr16(&Vt[r0 * D + 8 * (c ^ pf_vswz<D>(r0)) + e]);
            const s16x4 hi4 = lds_read_tr16(&Vt[r1 * D + 8 * (c ^ pf_vswz<D>(r1)) + e]);
            o[dt] = mfma32x32x16<BF16>(concat4(lo, hi4), pb, o[dt]);
        }
    };
    // Move m (and rescale O and l) for rows whose tile max passed m + margin.
    auto rescale = [&](float mx) {
        const float m_cand = mx * p.c;
        const bool grow = m_cand > m_i + kLazyRescale;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = grow ? m_cand : m_i;
            const float alpha = fast_exp2(m_i - m_new);
            m_i = m_new;
            l_i *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
            return true;
        }
        return false;
    };

    // One key tile. The probabilities of keys 0..31 are computed with the
    // current m while the QK MFMAs of keys 32..63 run; if the tile's max then
    // moves m (rare after the first tile), they are recomputed before any P V.
    // The exps of keys 32..63 run alongside the P V MFMAs of keys 0..31.
    auto tile = [&](const uint16_t* Kt, const uint16_t* Vt, int kv0, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        f32x16 s0, s1;
        s16x8 pb[4];
        qk_half(s0, Kt, 0);
        if constexpr (!FULL) mask_half(s0, kv0, 0);
        qk_half(s1, Kt, 1);
        float psum0 = softmax_half(s0, pb[0], pb[1]);
        if constexpr (FULL) {
            sched_group<0x100, 2>();
#pragma unroll
            for (int i = 0; i < D / 16; ++i) {
                sched_group<0x008, 1>();
                if (i + 2 < D / 16) sched_group<0x100, 1>();
                sched_group<0x002, 56 / (D / 16) + 1>();
            }
        }
        if constexpr (!FULL) mask_half(s1, kv0, 1);
        const float mx = max_with_other_half(fmaxf(max_half(s0), max_half(s1)));
        if (rescale(mx)) psum0 = softmax_half(s0, pb[0], pb[1]);
        pv_chunk(pb[0], Vt, 0);
        pv_chunk(pb[1], Vt, 1);
        const float psum1 = softmax_half(s1, pb[2], pb[3]);
        pv_chunk(pb[2], Vt, 2);
        pv_chunk(pb[3], Vt, 3);
        if constexpr (FULL) {
            sched_group<0x100, 4>();
#pragma unroll
            for (int i = 0; i < 4 * NDT; ++i) {
                sched_group<0x008, 1>();
                if (i + 2 < 4 * NDT) sched_group<0x100, 2>();
                if (i < 2 * NDT) sched_group<0x002, 56 / (2 * NDT) + 1>();
            }
        }
        l_i += psum0 + psum1;
    };

    // Key tile t lives in buffer (t - j_begin) % 2; tile j+1 is requested while
    // tile j is used, then one wait and one barrier per tile.
    auto iter = [&](int j, const uint16_t* Kc, const uint16_t* Vc, uint16_t* Kl, uint16_t* Vl) {
        load_k_tile(Kl, j + 1);
        load_v_tile(Vl, j + 1);
        if (!tile_empty(j)) {
            if (tile_full(j)) tile(Kc, Vc, j * PF_BN, BoolC<true>{});
            else tile(Kc, Vc, j * PF_BN, BoolC<false>{});
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    const int nt = j_end - j_begin;
    if (nt > 0) {
        load_k_tile(Ks0, j_begin);
        load_v_tile(Vs0, j_begin);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }
    for (int r = 0; r < nt; r += 2) {
        iter(j_begin + r, Ks0, Vs0, Ks1, Vs1);
        if (r + 1 < nt) iter(j_begin + r + 1, Ks1, Vs1, Ks0, Vs0);
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
