// Device-side helpers shared by the gfx950 kernels of the fast-weight delta-rule layer.
// Types, bf16 <-> fp32 conversion, element loads/stores for the two I/O element types, and
// thin wrappers over the two MFMA shapes the kernels use.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fwa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16;

constexpr float kDpfpEps = 1e-6f;  // [FWT] "DPFP / normalisation": added to the sum

__device__ __forceinline__ float bf16_bits_to_f32(u16 h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ u16 f32_to_bf16_bits(float f) {
    __bf16 b = static_cast<__bf16>(f);
    return __builtin_bit_cast(u16, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v;
    v[0] = static_cast<__bf16>(lo);
    v[1] = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, v);
}

// Element I/O for the caller's dtype (fp32 or bf16 storage).
template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
    if constexpr (BF16) return bf16_bits_to_f32(static_cast<const u16*>(p)[i]);
    else return static_cast<const float*>(p)[i];
}

template <bool BF16>
__device__ __forceinline__ void store_elem(void* p, int64_t i, float v) {
    if constexpr (BF16) static_cast<u16*>(p)[i] = f32_to_bf16_bits(v);
    else static_cast<float*>(p)[i] = v;
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(u16 h) { return bf16_bits_to_f32(h); }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ u16 from_f32<u16>(float x) { return f32_to_bf16_bits(x); }

__device__ __forceinline__ float relu(float x) { return x > 0.0f ? x : 0.0f; }

// sigmoid evaluated so that neither branch overflows; sigmoid(-inf) = 0, sigmoid(+inf) = 1.
__device__ __forceinline__ float sigmoid_stable(float x) {
    if (x >= 0.0f) return 1.0f / (1.0f + expf(-x));
    float e = expf(x);
    return e / (1.0f + e);
}

// D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16).
// Lane l holds A[l%16][8*(l/16) + s] and B[8*(l/16) + s][l%16] in slot s; the result holds
// D[4*(l/16) + r][l%16] in slot r.
__device__ __forceinline__ f32x4 mfma_bf16_k32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(16x16 fp32) += A(16x4 fp32) * B(4x16 fp32).
// Lane l holds A[l%16][l/16] and B[l/16][l%16]; the result layout is as above.
__device__ __forceinline__ f32x4 mfma_f32_k4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16 lanes, lane i
// receives in slot e the (i % 4)-th 16-bit element of the 8 bytes addressed by lane
// 4 e + i / 4 of the group.  `p` must point into LDS and be 8-byte aligned.
__device__ __forceinline__ bf16x4 lds_read_tr_b16x4(const void* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const_cast<void*>(p)));
    return __builtin_bit_cast(bf16x4, r);
}

// One 8-byte LDS read that the compiler does not pair with another into ds_read2_b64: the
// element offset passes through an empty asm statement (no instruction), so no two reads share
// a base register.  On gfx950 a paired read costs about twice the LDS cycles of two single
// 8-byte reads, and twice that again when the halves of the pair meet on the same banks.
__device__ __forceinline__ bf16x4 lds_read_b64_single(const u16* base, int off) {
    __asm__("" : "+v"(off));
    return *reinterpret_cast<const bf16x4*>(base + off);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.0f, 0.0f, 0.0f, 0.0f}; }

// x from another lane of the same 16-lane row, selected by a DPP control (compile-time).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of 8 lanes, in every lane of the group, by DPP (no LDS traffic):
// lane ^ 1, lane ^ 2 (quad permutes), then the mirrored lane of the other quad.
__device__ __forceinline__ float sum8_dpp(float x) {
    x += dpp_f32<0xB1>(x);
    x += dpp_f32<0x4E>(x);
    return x + dpp_f32<0x141>(x);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations, not for its
// global loads and stores in flight.  The kernels here share data inside a workgroup through
// LDS alone, so a barrier never has to drain prefetched loads or the stores of results that
// only later kernels read.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup placement.  Workgroups are dispatched to the 8 XCDs round robin by index; when
// B*H is a multiple of 8, all workgroups of (b, h) go to XCD (b*H + h) mod 8 in all three
// kernels, so the chain and output kernels find the prep kernel's results in that XCD's L2.
// Maps a workgroup index to (bh, i), i = index among the workgroups of bh (per_bh of them).
struct BhIndex {
    int bh;
    int64_t i;
};
__device__ __forceinline__ BhIndex xcd_local(int64_t b, int BH, int64_t per_bh) {
    if (((b | per_bh) >> 32) == 0) {
        // workgroup indices fit 32 bits (a uniform branch): 32-bit division is a few
        // instructions, the 64-bit one about a hundred
        const uint32_t bb = static_cast<uint32_t>(b), pb = static_cast<uint32_t>(per_bh);
        if ((BH & 7) == 0) {
            const uint32_t x = bb & 7, j = bb >> 3, q = j / pb;
            return BhIndex{static_cast<int>(q * 8 + x), static_cast<int64_t>(j - q * pb)};
        }
        const uint32_t q = bb / pb;
        return BhIndex{static_cast<int>(q), static_cast<int64_t>(bb - q * pb)};
    }
    if ((BH & 7) == 0) {
        const int64_t x = b & 7, j = b >> 3;      // XCD and index inside it
        return BhIndex{static_cast<int>((j / per_bh) * 8 + x), j % per_bh};
    }
    return BhIndex{static_cast<int>(b / per_bh), b % per_bh};
}

}  // namespace fwa
