// state_update.hip -- one-token selective state update (the recurrent / decode form of the
// selective scan) for gfx950.
//
// Per (b, d), with the state updated in place:
//   delta = softplus(dt + dt_bias_d)
//   h[n]  = exp(delta A_dn) h[n] + delta B_bn x        (Euler input term, as in the scan)
//   out   = (sum_n C_bn h[n] + D_d x) silu(z)
// This is the loop body of the Keras/TensorFlow tutorial's `selective_scan` recurrence for a
// single token; the mamba-jax README (`--scan` generation) and the upstream README
// (generation benchmarks) run the model this way, one token at a time.
//
// The step reads and writes the (batch, d_inner, 16) fp32 state once and is bound by memory
// traffic.  Four lanes share a row (16 B of state each, so a wavefront covers 1 KiB of
// contiguous state per access); the partial C.h sums meet through two DPP quad-permute adds.
#include "device_math.hpp"
#include "mss_internal.hpp"

namespace mss {
namespace {

struct DArgs {
    float* state;
    const void* x;
    const void* dt;
    const void* z;
    const float* A;
    const float* B;
    const float* C;
    const float* D;
    const float* bias;
    void* out;
    int64_t Dn, rows;
};

__device__ __forceinline__ float quad_sum(float v) {
    // quad_perm [1,0,3,2] then [2,3,0,1]: every lane of the quad ends with the quad's sum
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    return v;
}

// Threads stride over the rows' quads (the grid is capped: a dispatch holds at most 2^32 - 1
// work-items per dimension).  The stride is a multiple of four, so the four lanes of a row stay
// together in every iteration and the quad's DPP sum sees only its own row.
template <class E, bool HAS_Z>
__global__ __launch_bounds__(256) void state_update_kernel(DArgs a) {
    const int64_t total = a.rows * 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gt < total; gt += stride) {
        const int64_t row = gt >> 2;   // flat (b, d)
        const int q = static_cast<int>(gt & 3);  // this lane holds states 4q .. 4q + 3
        const int64_t d = row % a.Dn;
        const int64_t b = row / a.Dn;
        const float xv = E::load1(a.x, row);
        const float dl = softplus(E::load1(a.dt, row) + (a.bias ? a.bias[d] : 0.0f));
        float4* sp = reinterpret_cast<float4*>(a.state) + row * 4 + q;
        const float4 s = *sp;
        const float4 A4 = reinterpret_cast<const float4*>(a.A)[d * 4 + q];
        const float4 B4 = reinterpret_cast<const float4*>(a.B)[b * 4 + q];
        const float4 C4 = reinterpret_cast<const float4*>(a.C)[b * 4 + q];
        const float dx = dl * xv;
        float4 hn;
        hn.x = fmaf(fast_exp2(dl * (A4.x * kLog2e)), s.x, dx * B4.x);
        hn.y = fmaf(fast_exp2(dl * (A4.y * kLog2e)), s.y, dx * B4.y);
        hn.z = fmaf(fast_exp2(dl * (A4.z * kLog2e)), s.z, dx * B4.z);
        hn.w = fmaf(fast_exp2(dl * (A4.w * kLog2e)), s.w, dx * B4.w);
        *sp = hn;
        float y = fmaf(C4.w, hn.w, fmaf(C4.z, hn.z, fmaf(C4.y, hn.y, C4.x * hn.x)));
        y = quad_sum(y);
        if (q == 0) {
            float o = fmaf(a.D ? a.D[d] : 0.0f, xv, y);
            if (HAS_Z) o *= silu(E::load1(a.z, row));
            E::store1(a.out, row, o);
        }
    }
}

template <class E, bool HAS_Z>
hipError_t launch_t(const DArgs& k, hipStream_t stream) {
    const int64_t threads = k.rows * 4;
    int64_t blocks = (threads + 255) / 256;
    if (blocks > (1 << 22)) blocks = 1 << 22;
    state_update_kernel<E, HAS_Z><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(k);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_state_update(const DecodeLaunch& a, hipStream_t stream) {
    DArgs k;
    k.state = a.state; k.x = a.x; k.dt = a.dt; k.z = a.z; k.A = a.A; k.B = a.B; k.C = a.C;
    k.D = a.D; k.bias = a.bias; k.out = a.out; k.Dn = a.Dn; k.rows = a.Bt * a.Dn;
    if (k.rows == 0) return hipSuccess;
    const bool hz = a.z != nullptr;
    if (a.bf16) return hz ? launch_t<BF16, true>(k, stream) : launch_t<BF16, false>(k, stream);
    return hz ? launch_t<F32, true>(k, stream) : launch_t<F32, false>(k, stream);
}

}  // namespace mss
