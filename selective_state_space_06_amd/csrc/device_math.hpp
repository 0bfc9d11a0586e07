// device_math.hpp -- element helpers shared by the gfx950 kernels of libmamba_scan.
//
// exp is evaluated as exp2 of a log2(e)-prescaled argument (one v_exp_f32), log as
// log2 (v_log_f32) times ln 2, reciprocals with v_rcp_f32.  bf16 <-> f32 conversions use
// the gfx950 hardware convert (round to nearest even) and a 16-bit shift.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mss {

// A native 4 x f32 vector (what the nontemporal builtins take; HIP's float4 is a struct).
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(w), w = e^-|x| in (0, 1].
// log1p(w) is taken as log(s) - ((s - 1) - w) with s = fl(1 + w): s - 1 is exact for
// s in [1, 2], so (s - 1) - w is exactly the rounding error e of s, and
// log(1 + w) = log(s) - e / s + O(e^2).  Dropping the 1/s costs at most |e| w / (1 + w),
// below 1e-7 relative to log1p(w), and keeps the small-w end (very negative x, where a
// plain log(1 + e^x) would lose most digits) accurate.
__device__ __forceinline__ float softplus(float x) {
    const float w = fast_exp2(-fabsf(x) * kLog2e);
    const float s = 1.0f + w;
    const float e = (s - 1.0f) - w;
    return fmaxf(x, 0.0f) + fmaf(fast_log2(s), kLn2, -e);
}

// silu(v) = v * sigmoid(v) = v / (1 + e^-v).  For v << 0, e^-v overflows to +inf and the
// reciprocal gives 0, the correct limit.
__device__ __forceinline__ float silu(float v) {
    return v * fast_rcp(1.0f + fast_exp2(-v * kLog2e));
}

// The scale of one step in the forward kernels' scaled state form (S4D power path): the lane
// keeps g = h / sc and step t takes s_t = x_t + copysign(2^-40, x_t), never zero, so B enters
// the state update without a multiplication by x.  The addition is kept apart from the
// multiplication that formed x (no fused multiply-add), so every kernel variant forms the same
// s from the same x.
constexpr float kScaleEps = 0x1p-40f;
__device__ __forceinline__ float step_scale(float x) {
#pragma clang fp contract(off)
    return x + copysignf(kScaleEps, x);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// Two floats -> one word holding two bf16 (lo = a, hi = b), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    bf2 v;
    v.x = static_cast<__bf16>(a);
    v.y = static_cast<__bf16>(b);
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float a) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
}

// Element type traits for the two storage types of u / delta / z / out.
struct F32 {
    using storage = float;
    static constexpr int kPerVec = 4;  // elements per 16-byte vector
    __device__ static float load1(const void* p, int64_t i) {
        return static_cast<const float*>(p)[i];
    }
    __device__ static void store1(void* p, int64_t i, float v) { static_cast<float*>(p)[i] = v; }
    // 16 bytes -> kPerVec floats
    __device__ static void unpack(const uint4& w, float* v) {
        v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y);
        v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
    }
    __device__ static uint4 pack(const float* v) {
        return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]),
                          __float_as_uint(v[2]), __float_as_uint(v[3]));
    }
    // element e (compile-time after unrolling) of a 16-byte vector
    __device__ static float elem(const uint4& w, int e) {
        const uint32_t x = e == 0 ? w.x : e == 1 ? w.y : e == 2 ? w.z : w.w;
        return __uint_as_float(x);
    }
};

struct BF16 {
    using storage = uint16_t;
    static constexpr int kPerVec = 8;
    __device__ static float load1(const void* p, int64_t i) {
        return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    }
    __device__ static void store1(void* p, int64_t i, float v) {
        static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
    }
    __device__ static void unpack(const uint4& w, float* v) {
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
        v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
    }
    __device__ static uint4 pack(const float* v) {
        return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                          pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    }
    __device__ static float elem(const uint4& w, int e) {
        const uint32_t x = (e >> 1) == 0 ? w.x : (e >> 1) == 1 ? w.y : (e >> 1) == 2 ? w.z : w.w;
        return (e & 1) ? bf16_hi(x) : bf16_lo(x);
    }
};

}  // namespace mss
