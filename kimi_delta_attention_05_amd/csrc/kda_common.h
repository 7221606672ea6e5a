// Internal helpers shared by the libkda kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 128;          // K = V = 128 (the contract's only head size)
constexpr float kL2Eps = 1e-6f;        // q/k L2 normalisation epsilon
constexpr float kLog2e = 1.4426950408889634f;

// ---- element conversion ------------------------------------------------------

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) {
    return static_cast<__bf16>(x);      // round to nearest even
}
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) {
    return static_cast<_Float16>(x);    // round to nearest even
}

// 2^x and 1/x on the hardware transcendental unit.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Logistic function for any finite x: exp2 of a non-positive argument only.
__device__ __forceinline__ float sigmoid_f(float x) {
    float z = fast_exp2(-fabsf(x) * kLog2e);          // in (0, 1]
    float r = fast_rcp(1.0f + z);
    return x >= 0.0f ? r : z * r;
}

// Workgroup barrier that orders LDS only: this wave's LDS operations complete,
// then all waves meet. __syncthreads() also fences global memory, which on gfx9
// waits for every outstanding global load, store and global->LDS copy
// (vmcnt(0)); the kernels here communicate within a workgroup through LDS
// only, so prefetches and output stores stay in flight across barriers. The
// "memory" clobbers keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until this wave's outstanding global loads (including global->LDS
// copies) have landed. Issued through the builtin (gfx9 encoding: vmcnt = 0,
// expcnt and lgkmcnt left at their maxima) rather than inline asm, so that the
// compiler's own wait insertion sees it and does not add another vmcnt(0)
// before the next LDS read of copied data, which would also wait for every
// store issued since.
__device__ __forceinline__ void wait_vmem() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("" ::: "memory");
}

// The same, except that the N newest vector memory operations of this wave may
// still be in flight (loads and stores complete in issue order for this counter).
template <int N>
__device__ __forceinline__ void wait_vmem_except() {
    static_assert(N >= 0 && N < 16, "vmcnt immediate (low field)");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);
    asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// Asynchronous copies from global memory straight into LDS (global->LDS DMA,
// no registers); completion is tracked by vmcnt like any vector load.
//
// A buffer resource for the byte range [base, base + bytes) (gfx9 word-3 format
// bits); a read outside the range returns zeros instead of faulting.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}

// buffer_load_dword{,x4} ... lds: lane i reads rsrc + voffset_i + soffset and
// writes lds_wave_base + SIZE * i, so a wave fills one contiguous block;
// lds_wave_base, rsrc and soffset must be wave-uniform. Issued as inline asm
// (M0, which addresses the LDS side, is saved and restored around it): the
// compiler then does not see an LDS write in flight and adds no vmcnt waits of
// its own before later LDS accesses. Every reader of the copied bytes waits
// explicitly (wait_vmem, then a barrier).
template <int SIZE>
__device__ __forceinline__ void buffer_copy_to_lds(const i32x4 &r, uint32_t voffset, uint32_t soffset,
                                                   const void *lds_wave_base) {
    const uint32_t la = (uint32_t)(uintptr_t)(lds_ptr_t)lds_wave_base;
    uint32_t saved;
    if constexpr (SIZE == 16)
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %4\n\ts_nop 0\n\t"
                     "buffer_load_dwordx4 %1, %2, %3 offen lds\n\ts_mov_b32 m0, %0"
                     : "=&s"(saved) : "v"(voffset), "s"(r), "s"(soffset), "s"(la) : "memory");
    else
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %4\n\ts_nop 0\n\t"
                     "buffer_load_dword %1, %2, %3 offen lds\n\ts_mov_b32 m0, %0"
                     : "=&s"(saved) : "v"(voffset), "s"(r), "s"(soffset), "s"(la) : "memory");
}
__device__ __forceinline__ void copy16_to_lds(const i32x4 &r, uint32_t voffset, uint32_t soffset,
                                              void *lds_wave_base) {
    buffer_copy_to_lds<16>(r, voffset, soffset, lds_wave_base);
}
__device__ __forceinline__ void copy4_to_lds(const i32x4 &r, uint32_t voffset, uint32_t soffset,
                                             void *lds_wave_base) {
    buffer_copy_to_lds<4>(r, voffset, soffset, lds_wave_base);
}

// 8 consecutive input elements kept in their storage format (prefetch buffers).
template <typename T> struct Vec8;
template <> struct Vec8<__bf16> {
    bf16x8 v;
    __device__ __forceinline__ void load(const __bf16 *p) { v = *(const bf16x8 *)p; }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)0.0f;
    }
    __device__ __forceinline__ float operator[](int e) const { return (float)v[e]; }
    __device__ __forceinline__ void store(__bf16 *p) const { *(bf16x8 *)p = v; }
};
template <> struct Vec8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = ((const f32x4 *)p)[0];
        b = ((const f32x4 *)p)[1];
    }
    __device__ __forceinline__ void zero() { a = f32x4{0.f, 0.f, 0.f, 0.f}; b = a; }
    __device__ __forceinline__ float operator[](int e) const { return e < 4 ? a[e] : b[e - 4]; }
    __device__ __forceinline__ void store(float *p) const {
        ((f32x4 *)p)[0] = a;
        ((f32x4 *)p)[1] = b;
    }
};

// ---- cross-lane reductions ---------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the sum.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp_f<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp_f<0x141>(x);   // row_half_mirror
    x += dpp_f<0x140>(x);   // row_mirror
    return x;
}

// Max of |x| over the 16 lanes of a DPP row.
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));
    x = fmaxf(x, dpp_f<0x4E>(x));
    x = fmaxf(x, dpp_f<0x141>(x));
    x = fmaxf(x, dpp_f<0x140>(x));
    return x;
}

// Max over all 64 lanes of the wave (every lane gets it).
__device__ __forceinline__ float wave_max(float x) {
    x = row16_max(x);
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}

// Max over the 64 lanes of a non-negative x, returned wave-uniform. For
// non-negative IEEE floats the unsigned order of the bit patterns is the
// numeric order, so the cross-lane part runs on integers: DPP within each row
// of 16 lanes, then the four row maxima through scalar registers (no LDS
// round trip).
__device__ __forceinline__ float wave_max_nonneg(float x) {
    uint32_t u = __float_as_uint(x);
    u = max(u, dpp_u<0xB1>(u));     // quad_perm [1,0,3,2]
    u = max(u, dpp_u<0x4E>(u));     // quad_perm [2,3,0,1]
    u = max(u, dpp_u<0x141>(u));    // row_half_mirror
    u = max(u, dpp_u<0x140>(u));    // row_mirror
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)u, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)u, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)u, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)u, 48);
    return __uint_as_float(max(max(a, b), max(c, d)));
}

__device__ __forceinline__ float wave_sum(float x) {
    x = row16_sum(x);
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// ---- MFMA 16x16x32 -----------------------------------------------------------
//
// A fragment: lane l holds row (l % 16) and 8 k-values; B fragment: lane l holds
// column (l % 16) and 8 k-values; lanes l and l' with the same l / 16 pair their
// k-values position by position, so any fixed assignment of logical k to
// (l / 16, position) gives the same product. Accumulator: lane l holds
// D[4 * (l / 16) + i][l % 16] for i = 0..3.
//
// The k order used throughout libkda for operands that also come out of an
// accumulator is  k(g, e) = (e < 4) ? 4g + e : 16 + 4g + (e - 4)  within each
// 32-wide k-step, g = l / 16: it is exactly what two vertically stacked 16x16
// accumulator tiles hold in one lane.

__device__ __forceinline__ int kperm(int g, int e) {
    return (e < 4) ? (4 * g + e) : (16 + 4 * g + (e - 4));
}

// Key channels follow a different order, chosen so that each lane's 8 channels
// of a k-step are contiguous in memory (one 16-byte load of bf16 inputs): the
// channel at k-index (g, e) of step s is 32 s + 8 g + e. Accumulator tiles
// whose rows are key channels (the state S^T, kg^T) therefore hold, in tile kb,
// row r = 4 g + i, the channel tile_chan(kb, r) below -- two consecutive tiles
// 2s, 2s+1 stack into exactly the k-step s operand order.
__device__ __forceinline__ int tile_chan(int kb, int r) {
    return 32 * (kb >> 1) + 8 * (r >> 2) + 4 * (kb & 1) + (r & 3);
}

__device__ __forceinline__ f32x4 mfma_f16(const float (&a)[8], const float (&b)[8], f32x4 acc) {
    half8 ha, hb;
#pragma unroll
    for (int e = 0; e < 8; ++e) { ha[e] = (_Float16)a[e]; hb[e] = (_Float16)b[e]; }
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(ha, hb, acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_h(const half8 &a, const half8 &b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}

// Three-product bf16 split: x = hi + lo with hi = bf16(x), lo = bf16(x - hi);
// a.b ~= ah.bh + ah.bl + al.bh (relative error ~2^-16, full fp32 exponent range).
__device__ __forceinline__ f32x4 mfma_x3(const float (&a)[8], const float (&b)[8], f32x4 acc) {
    bf16x8 ah, al, bh, bl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        __bf16 t = (__bf16)a[e]; ah[e] = t; al[e] = (__bf16)(a[e] - (float)t);
        __bf16 u = (__bf16)b[e]; bh[e] = u; bl[e] = (__bf16)(b[e] - (float)u);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
    return acc;
}

// fp32 product on the fp32 MFMA (v_mfma_f32_16x16x4f32): each of the 8
// positions is one 4-deep step across the four lane groups, so the 8 calls
// together cover the same 32 k-values in the same pairing as above.
__device__ __forceinline__ f32x4 mfma_f32x8(const float (&a)[8], const float (&b)[8], f32x4 acc) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
    return acc;
}

// 8 consecutive elements as fp32 (16- or 32-byte vector loads).
__device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
    const f32x4 a = ((const f32x4 *)p)[0], b = ((const f32x4 *)p)[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[e + 4] = b[e]; }
}
__device__ __forceinline__ void load8(const __bf16 *p, float (&x)[8]) {
    const bf16x8 a = *(const bf16x8 *)p;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)a[e];
}

// 8 fp32 values stored as 8 consecutive elements (one 16- or 32-byte store;
// bf16 rounds to nearest even).
template <typename T>
__device__ __forceinline__ void store8(T *p, const float (&x)[8]);
template <>
__device__ __forceinline__ void store8<float>(float *p, const float (&x)[8]) {
    ((f32x4 *)p)[0] = f32x4{x[0], x[1], x[2], x[3]};
    ((f32x4 *)p)[1] = f32x4{x[4], x[5], x[6], x[7]};
}
template <>
__device__ __forceinline__ void store8<__bf16>(__bf16 *p, const float (&x)[8]) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)x[e];
    *(bf16x8 *)p = v;
}

// The same as store8 with a non-temporal hint: for outputs that no later
// access of the same kernel reads (streamed to HBM instead of kept in cache).
template <typename T>
__device__ __forceinline__ void store8_nt(T *p, const float (&x)[8]);
template <>
__device__ __forceinline__ void store8_nt<float>(float *p, const float (&x)[8]) {
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, (f32x4 *)p);
    __builtin_nontemporal_store(f32x4{x[4], x[5], x[6], x[7]}, (f32x4 *)p + 1);
}
template <>
__device__ __forceinline__ void store8_nt<__bf16>(__bf16 *p, const float (&x)[8]) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)x[e];
    __builtin_nontemporal_store(v, (bf16x8 *)p);
}

// Power of two 2^e with e = ceil(log2(m)) - target, so that m * 2^-e <= 2^target;
// returns 1 for m == 0 or non-finite m.
__device__ __forceinline__ float pow2_scale_for(float m, int target) {
    if (!(m > 0.0f) || !(m < 3.0e38f)) return 1.0f;
    int e = ((int)((__float_as_uint(m) >> 23) & 0xFF)) - 127 + 1 - target;
    e = e < -126 ? -126 : (e > 127 ? 127 : e);
    return __uint_as_float((uint32_t)(e + 127) << 23);
}

}  // namespace kda
