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
// bound by memory traffic.  N / 4 lanes share a row, one 16-byte vector of states each, so the 64
// lanes of a wave cover 64 / (N / 4) whole consecutive rows: every load and store of the state is
// one contiguous KiB.  The partial C.h sums meet through DPP quad-permute adds and, for N > 16,
// lane-exchange adds across the quads of the row.
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

// Sum over the LR lanes of a row (LR = 4, 8, 16 or 32 consecutive lanes, aligned): every lane of
// the row ends with the row's sum.
template <int LR>
__device__ __forceinline__ float row_sum(float v) {
    v = quad_sum(v);
    if (LR >= 8) v += __shfl_xor(v, 4);
    if (LR >= 16) v += __shfl_xor(v, 8);
    if (LR >= 32) v += __shfl_xor(v, 16);
    return v;
}

// Threads stride over the rows' lanes (the grid is capped: a dispatch holds at most 2^32 - 1
// work-items per dimension).  The stride is a multiple of LR, so the lanes of a row stay together
// in every iteration and the row sum sees only its own row; lane k of a row holds states
// 4 k .. 4 k + 3.  Each thread takes kItems rows per round, one stride apart, and issues all their
// loads before any arithmetic: the step is bound by the latency of its state reads, and this
// doubles the reads in flight (64 x 5120 states in HBM: 12.4 -> 12.0 us at N = 16; four items
// were slower at every N).  An item past the end re-reads the round's first row and stores
// nothing; a row is valid or invalid as a whole, so the sums of valid rows see only valid lanes.
constexpr int kItems = 2;

template <class E, bool HAS_Z, int N>
__global__ __launch_bounds__(256) void state_update_kernel(DArgs a) {
    constexpr int LR = N / 4;  // lanes per row
    constexpr int IT = kItems;
    const int64_t total = a.rows * LR;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int k = static_cast<int>(threadIdx.x & (LR - 1));
    const float4* st4 = reinterpret_cast<const float4*>(a.state);
    const float4* A4p = reinterpret_cast<const float4*>(a.A);
    const float4* B4p = reinterpret_cast<const float4*>(a.B);
    const float4* C4p = reinterpret_cast<const float4*>(a.C);
    for (int64_t g0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g0 < total; g0 += IT * stride) {
        int64_t row[IT], d[IT];
        bool ok[IT];
        float xv[IT], dtv[IT], zv[IT], bias[IT];
        float4 s[IT], A4[IT], B4[IT], C4[IT];
#pragma unroll
        for (int u = 0; u < IT; ++u) {
            const int64_t gt = g0 + u * stride;
            ok[u] = gt < total;
            row[u] = (ok[u] ? gt : g0) / LR;  // flat (b, d)
            d[u] = row[u] % a.Dn;
            const int64_t b = row[u] / a.Dn;
            xv[u] = E::load1(a.x, row[u]);
            dtv[u] = E::load1(a.dt, row[u]);
            zv[u] = HAS_Z ? E::load1(a.z, row[u]) : 0.0f;
            bias[u] = a.bias ? a.bias[d[u]] : 0.0f;
            s[u] = st4[row[u] * LR + k];
            A4[u] = A4p[d[u] * LR + k];
            B4[u] = B4p[b * LR + k];
            C4[u] = C4p[b * LR + k];
        }
#pragma unroll
        for (int u = 0; u < IT; ++u) {
            const float dl = softplus(dtv[u] + bias[u]);
            const float dx = dl * xv[u];
            float4 hn;
            hn.x = fmaf(fast_exp2(dl * (A4[u].x * kLog2e)), s[u].x, dx * B4[u].x);
            hn.y = fmaf(fast_exp2(dl * (A4[u].y * kLog2e)), s[u].y, dx * B4[u].y);
            hn.z = fmaf(fast_exp2(dl * (A4[u].z * kLog2e)), s[u].z, dx * B4[u].z);
            hn.w = fmaf(fast_exp2(dl * (A4[u].w * kLog2e)), s[u].w, dx * B4[u].w);
            if (ok[u]) reinterpret_cast<float4*>(a.state)[row[u] * LR + k] = hn;
            float y = fmaf(C4[u].w, hn.w, fmaf(C4[u].z, hn.z, fmaf(C4[u].y, hn.y, C4[u].x * hn.x)));
            y = row_sum<LR>(y);
            if (k == 0 && ok[u]) {
                float o = fmaf(a.D ? a.D[d[u]] : 0.0f, xv[u], y);
                if (HAS_Z) o *= silu(zv[u]);
                E::store1(a.out, row[u], o);
            }
        }
    }
}

template <class E, bool HAS_Z, int N>
hipError_t launch_t(const DArgs& k, hipStream_t stream) {
    const int64_t threads = k.rows * (N / 4);
    int64_t blocks = (threads + 256 * kItems - 1) / (256 * kItems);
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
