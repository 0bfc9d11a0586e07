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
// The step reads and writes the (batch, d_inner, N) fp32 state once (N = 16, 32, 64 or 128) and is
// bound by memory traffic.  Four lanes share a row (N / 4 states each, 16 B per access, a row's
// four lanes covering 64 contiguous bytes); the partial C.h sums meet through two DPP quad-permute
// adds.
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
// together in every iteration and the quad's DPP sum sees only its own row.  Lane q of a row holds
// the states 4 (4 v + q) .. + 3 for v < N / 16 (each 16-byte load of the row's four lanes covers 64
// contiguous bytes).  For N = 16 each thread takes kItems quads per round, one stride apart, and
// issues all their loads before any arithmetic: the step is bound by the latency of its state
// reads, and this doubles the reads in flight.  (An item past the end re-reads the round's first
// quad and stores nothing; a quad is valid or invalid as a whole, so the DPP sums of valid rows
// see only valid lanes.)
constexpr int kItems = 2;

template <class E, bool HAS_Z, int N>
__global__ __launch_bounds__(256) void state_update_kernel(DArgs a) {
    constexpr int VQ = N / 16;                  // 16-byte vectors of a row per lane
    constexpr int IT = N == 16 ? kItems : 1;    // quads per thread and round
    const int64_t total = a.rows * 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int q = static_cast<int>(threadIdx.x & 3);
    const float4* st4 = reinterpret_cast<const float4*>(a.state);
    const float4* A4p = reinterpret_cast<const float4*>(a.A);
    const float4* B4p = reinterpret_cast<const float4*>(a.B);
    const float4* C4p = reinterpret_cast<const float4*>(a.C);
    for (int64_t g0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g0 < total; g0 += IT * stride) {
        int64_t row[IT], d[IT];
        bool ok[IT];
        float xv[IT], dtv[IT], zv[IT], bias[IT];
        float4 s[IT][VQ], A4[IT][VQ], B4[IT][VQ], C4[IT][VQ];
#pragma unroll
        for (int u = 0; u < IT; ++u) {
            const int64_t gt = g0 + u * stride;
            ok[u] = gt < total;
            row[u] = (ok[u] ? gt : g0) >> 2;  // flat (b, d)
            d[u] = row[u] % a.Dn;
            const int64_t b = row[u] / a.Dn;
            xv[u] = E::load1(a.x, row[u]);
            dtv[u] = E::load1(a.dt, row[u]);
            zv[u] = HAS_Z ? E::load1(a.z, row[u]) : 0.0f;
            bias[u] = a.bias ? a.bias[d[u]] : 0.0f;
#pragma unroll
            for (int v = 0; v < VQ; ++v) {
                const int k = 4 * v + q;
                s[u][v] = st4[row[u] * (N / 4) + k];
                A4[u][v] = A4p[d[u] * (N / 4) + k];
                B4[u][v] = B4p[b * (N / 4) + k];
                C4[u][v] = C4p[b * (N / 4) + k];
            }
        }
#pragma unroll
        for (int u = 0; u < IT; ++u) {
            const float dl = softplus(dtv[u] + bias[u]);
            const float dx = dl * xv[u];
            float y = 0.0f;
#pragma unroll
            for (int v = 0; v < VQ; ++v) {
                float4 hn;
                hn.x = fmaf(fast_exp2(dl * (A4[u][v].x * kLog2e)), s[u][v].x, dx * B4[u][v].x);
                hn.y = fmaf(fast_exp2(dl * (A4[u][v].y * kLog2e)), s[u][v].y, dx * B4[u][v].y);
                hn.z = fmaf(fast_exp2(dl * (A4[u][v].z * kLog2e)), s[u][v].z, dx * B4[u][v].z);
                hn.w = fmaf(fast_exp2(dl * (A4[u][v].w * kLog2e)), s[u][v].w, dx * B4[u][v].w);
                if (ok[u]) reinterpret_cast<float4*>(a.state)[row[u] * (N / 4) + 4 * v + q] = hn;
                y = fmaf(C4[u][v].w, hn.w, fmaf(C4[u][v].z, hn.z, fmaf(C4[u][v].y, hn.y, fmaf(C4[u][v].x, hn.x, y))));
            }
            y = quad_sum(y);
            if (q == 0 && ok[u]) {
                float o = fmaf(a.D ? a.D[d[u]] : 0.0f, xv[u], y);
                if (HAS_Z) o *= silu(zv[u]);
                E::store1(a.out, row[u], o);
            }
        }
    }
}

template <class E, bool HAS_Z, int N>
hipError_t launch_t(const DArgs& k, hipStream_t stream) {
    constexpr int IT = N == 16 ? kItems : 1;
    const int64_t threads = k.rows * 4;
    int64_t blocks = (threads + 256 * IT - 1) / (256 * IT);
    if (blocks > (1 << 22)) blocks = 1 << 22;
    state_update_kernel<E, HAS_Z, N><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(k);
    return hipGetLastError();
}

template <class E, bool HAS_Z>
hipError_t launch_n(const DArgs& k, int N, hipStream_t stream) {
    switch (N) {
        case 16: return launch_t<E, HAS_Z, 16>(k, stream);
        case 32: return launch_t<E, HAS_Z, 32>(k, stream);
        case 64: return launch_t<E, HAS_Z, 64>(k, stream);
        default: return launch_t<E, HAS_Z, 128>(k, stream);
    }
}

}  // namespace

hipError_t launch_state_update(const DecodeLaunch& a, hipStream_t stream) {
    DArgs k;
    k.state = a.state; k.x = a.x; k.dt = a.dt; k.z = a.z; k.A = a.A; k.B = a.B; k.C = a.C;
    k.D = a.D; k.bias = a.bias; k.out = a.out; k.Dn = a.Dn; k.rows = a.Bt * a.Dn;
    if (k.rows == 0) return hipSuccess;
    const bool hz = a.z != nullptr;
    if (a.bf16) return hz ? launch_n<BF16, true>(k, a.N, stream) : launch_n<BF16, false>(k, a.N, stream);
    return hz ? launch_n<F32, true>(k, a.N, stream) : launch_n<F32, false>(k, a.N, stream);
}

}  // namespace mss
