// Device-side helpers shared by the attention kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
// Initial running max, in scaled log2 units: finite, so that the first
// rescale factor exp2(m_old - m_new) is exactly 0 instead of NaN.
constexpr float kMaxInit = -1.0e30f;
// Stand-in score for masked keys when reducing the tile max.
constexpr float kMaskedScore = -3.4028234663852886e38f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Instruction-scheduling hint for the device compiler: the next group of the
// current scheduling region holds N instructions of class MASK (0x002 VALU,
// 0x008 MFMA, 0x100 LDS read). It only shapes the order of independent
// instructions; the host pass of the compiler never sees it.
template <int MASK, int N>
__device__ __forceinline__ void sched_group() {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_sched_group_barrier(MASK, N, 0);
#endif
}

// Wait until at most N vector-memory operations of this wave are in flight
// (loads complete in issue order, so this waits for all but the last N).
// Emitted as the s_waitcnt builtin (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt and lgkmcnt left at their maxima) so that the compiler's own
// wait insertion knows about it, between two compiler memory barriers.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("" ::: "memory");
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
#endif
    asm volatile("" ::: "memory");
}

// Workgroup barrier for LDS tiles filled by direct-to-LDS loads. Unlike
// __syncthreads(), whose release fence makes the compiler wait for every
// outstanding load that writes LDS (vmcnt(0)) and so drains all prefetches at
// each barrier, this waits only for this wave's own LDS instructions
// (lgkmcnt(0): its reads are done before others overwrite the data, its
// writes are visible after the barrier); the caller waits for exactly the
// direct loads the barrier publishes (wait_vmcnt). The compiler memory
// barriers keep LDS accesses on their side of it.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("" ::: "memory");
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt at their maxima
    __builtin_amdgcn_s_barrier();
#endif
    asm volatile("" ::: "memory");
}

// Scheduling fence: the compiler moves no instruction across it.
__device__ __forceinline__ void sched_fence() {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_sched_barrier(0);
#endif
}

// max(max(a, b), c): with NaNs ignored (-fno-honor-nans) the compiler emits
// one v_max3_f32 per call when the calls are chained through the first
// argument. (Not inline asm: the compiler must see these reads, because they
// often consume MFMA results and need its hazard wait states.)
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Value of lane (l ^ 32) for every lane l, with one v_permlane32_swap.
__device__ __forceinline__ float max_with_other_half(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_other_half(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Attention sink (one extra logit without a value row, in scaled log2 units
// s2 = sink * log2 e) folded into a finished row with running max m and sum
// l (also log2 units): the max becomes max(m, s2), O and l are rescaled once
// to it and the sink's exponential joins the sum. Returns the factor for O
// and updates m and l. A sink of -inf (or none) leaves everything as it is.
// A row that saw no key (l = 0, m at its finite initial value) ends with
// l = 1, O = 0 and m = s2.
__device__ __forceinline__ float fold_sink(float s2, float& m, float& l) {
    if (!(s2 > -__builtin_inff())) return 1.f;
    const float mn = fmaxf(m, s2);
    const float a = __builtin_amdgcn_exp2f(m - mn);
    l = l * a + __builtin_amdgcn_exp2f(s2 - mn);
    m = mn;
    return a;
}

// A sink logit that is NaN or +inf (any non-finite value but -inf), tested on
// its bits: the kernels are built without NaN semantics for float compares.
// Such a sink makes every row of its head NaN (its exp is NaN or makes the
// sum infinite), so the epilogues then write NaN bit patterns directly.
__device__ __forceinline__ bool sink_gives_nan(float s) {
    const uint32_t bits = __float_as_uint(s);
    return (bits & 0x7f800000u) == 0x7f800000u && bits != 0xff800000u;
}
constexpr uint32_t kNaN32 = 0x7fc00000u;                // quiet f32 NaN
template <bool BF16>
constexpr uint32_t kNaN16x2 = BF16 ? 0x7fc07fc0u : 0x7e007e00u;  // two quiet bf16 / f16 NaNs

// Round-to-nearest-even conversions of f32 to 16-bit floats, returned as raw bits.
template <bool BF16>
__device__ __forceinline__ uint16_t f32_to_16(float x) {
    if constexpr (BF16) {
        __bf16 h = (__bf16)x;
        return __builtin_bit_cast(uint16_t, h);
    } else {
        _Float16 h = (_Float16)x;
        return __builtin_bit_cast(uint16_t, h);
    }
}
template <bool BF16>
__device__ __forceinline__ float f16bits_to_f32(uint16_t b) {
    if constexpr (BF16) {
        return __uint_as_float((uint32_t)b << 16);
    } else {
        return (float)__builtin_bit_cast(_Float16, b);
    }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two f32 -> one dword of two 16-bit floats (round to nearest even), low half first.
template <bool BF16>
__device__ __forceinline__ uint32_t pack2_16(float a, float b) {
    const f32x2 v = {a, b};
    if constexpr (BF16) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    } else {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    }
}

// acc + x.lo * y.lo + x.hi * y.hi with 16-bit float pairs (one v_dot2c_f32_*).
template <bool BF16>
__device__ __forceinline__ float dot2_16(uint32_t x, uint32_t y, float acc) {
    if constexpr (BF16) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y), acc, false);
    } else {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), __builtin_bit_cast(f16x2, y), acc, false);
    }
}

// 32x32x16 MFMA with f32 accumulation; operands are 8 16-bit values per lane.
template <bool BF16>
__device__ __forceinline__ f32x16 mfma32x32x16(s16x8 a, s16x8 b, f32x16 c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
}

// 16x16x32 MFMA with f32 accumulation.
template <bool BF16>
__device__ __forceinline__ f32x4 mfma16x16x32(s16x8 a, s16x8 b, f32x4 c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
}

// LDS transpose read: within each group of 16 lanes, lane i receives element
// i%4 of the 8-byte rows supplied by lanes 4j + i/4 (j = 0..3). With lane s
// of a group pointing at row (r0 + s/4), column (c0 + 4*(s%4)) of a row-major
// 16-bit matrix, lane i gets column c0 + i of rows r0..r0+3.
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

__device__ __forceinline__ s16x8 concat4(s16x4 a, s16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace attn
