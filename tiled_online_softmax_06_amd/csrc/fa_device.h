// fa_device.h — device-side helpers shared by the forward and backward
// kernels (gfx950 only): vector types, the MFMA wrappers, lane-pair
// reductions, the XCD-aware tile numbering, LDS swizzles and the global->LDS
// DMA.  Internal; included by the .hip kernel sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
// fp32 forward kernel: the reference max is raised only when a tile max
// exceeds it by more than this (log2 units), so weights stay <= 2^8.
constexpr float kRescaleSlack = 8.0f;
// Bound on one lane's sum of a tile's weights before the fp16/bf16 forward
// kernels raise their reference max: weights stay <= 2^12, inside fp16 range
// for the P.V operand.
constexpr float kTileSumLimit = 4096.0f;

template <typename T> struct Mfma;

template <> struct Mfma<__bf16> {
    using frag = bf16x8;
    static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(frag, a),
                                                       __builtin_bit_cast(frag, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ u32x4 pack(const float* p) {
        frag f;
#pragma unroll
        for (int t = 0; t < 8; ++t) f[t] = (__bf16)p[t];
        return __builtin_bit_cast(u32x4, f);
    }
    static __device__ __forceinline__ u32x2 pack4(const float* p) {
        __bf16 __attribute__((ext_vector_type(4))) f;
#pragma unroll
        for (int t = 0; t < 4; ++t) f[t] = (__bf16)p[t];
        return __builtin_bit_cast(u32x2, f);
    }
};

template <> struct Mfma<_Float16> {
    using frag = f16x8;
    static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(frag, a),
                                                      __builtin_bit_cast(frag, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ u32x4 pack(const float* p) {
        frag f;
#pragma unroll
        for (int t = 0; t < 8; ++t) f[t] = (_Float16)p[t];
        return __builtin_bit_cast(u32x4, f);
    }
    static __device__ __forceinline__ u32x2 pack4(const float* p) {
        _Float16 __attribute__((ext_vector_type(4))) f;
#pragma unroll
        for (int t = 0; t < 4; ++t) f[t] = (_Float16)p[t];
        return __builtin_bit_cast(u32x2, f);
    }
};

// Sum / max of the values held by lanes l and l^32 (the two lane halves that
// hold the same query).  permlane32_swap exchanges the halves of two copies;
// combining both results gives every lane the pair's sum / max.
__device__ __forceinline__ float pair_max(float x) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Workgroup id -> logical tile id.  Dispatch sends workgroup w to XCD w % 8;
// this bijection gives XCD x the contiguous logical range
// [x*per + min(x, rem), ... + per + (x < rem)).
__device__ __forceinline__ int xcd_tile(int wg, int total) {
    const int per = total >> 3, rem = total & 7;
    const int x = wg & 7, slot = wg >> 3;
    return x * per + min(x, rem) + slot;
}

// Key row held by accumulator register r in lane half `half` (D layout).
__device__ __forceinline__ int acc_row(int r, int half) {
    return 8 * (r >> 2) + 4 * half + (r & 3);
}

// ---------------------------------------------------------------------------
// fp16 / bf16 kernel
// ---------------------------------------------------------------------------

// LDS swizzles.  A K or V tile is stored row-major (key rows of D elements),
// each row split into 16-byte chunks; chunk c of row r sits at position
// c ^ f(r).  The DMA that fills LDS writes 1 KB per wave instruction
// contiguously (64 lanes x 16 bytes), so the swizzle is applied by choosing
// which global chunk each lane fetches.
//  * K is read as the A operand of S^T = K Q^T: 16 lanes read one chunk of 16
//    consecutive rows, so f must separate 16 consecutive rows.
//  * V is read with the LDS transpose read (ds_read_b64_tr_b16): 32 lanes read
//    4 consecutive rows x 4 consecutive chunks, so f must separate rows mod 4.
template <int D> __device__ __forceinline__ constexpr int swz_k(int r) {
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D> __device__ __forceinline__ constexpr int swz_v(int r) {
    return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

template <int N_> struct Int { static constexpr int value = N_; };

template <int B_, int E_, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B_ < E_) {
        f(Int<B_>{});
        static_for<B_ + 1, E_>(f);
    }
}

// 16-byte DMA from a buffer into LDS: lane l writes lds + 16*l (lds must be
// wave-uniform).  The builtin only exists in the device pass; the host pass
// must still see a body to emit the kernel's launch stub.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, char* lds, int voff, int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
#endif
}

}  // namespace
}  // namespace fa
