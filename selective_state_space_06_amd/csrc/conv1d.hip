// conv1d.hip -- causal depthwise conv1d (+ silu) in front of the scan, and its one-token form.
//
// The tutorial page's `MambaBlock` passes the scan input through a Keras Conv1D with one filter
// per channel (groups = channels), kernel_size 4, a bias, channels-first data and causal padding,
// then swish; the upstream README calls the width d_conv = 4.  A Keras Conv1D is a
// cross-correlation and causal padding puts K - 1 zeros on the left, so per channel d
//     y[t] = bias_d + sum_{k=0}^{K-1} w[d][k] x[t - (K-1) + k],     out = silu(y) (or y)
// with w[d][K-1] on the current input.  Here the K - 1 inputs before t = 0 may come from a
// carried state (chunked prefill) instead of zeros, and the last K - 1 inputs can be returned as
// the state for the next chunk or for the one-token step, which keeps them as a rolling window.
//
// Forward layout: one thread per 16-byte vector of a row, consecutive threads on consecutive
// vectors (a wave reads 1 KB of one row in one go), so the conv is a pure streaming kernel: each
// input read once from memory, each output written once.  A thread's K - 1 left neighbours are
// the tail of the previous vector, which the thread loads as well (its neighbour's line, already
// on its way); a row's first vector takes them from the carried state.
#include "device_math.hpp"
#include "mss_internal.hpp"

namespace mss {
namespace {

constexpr int kMaxK = 4;

struct ConvArgs {
    const void* x;
    const float* w;         // (Dn, K)
    const float* bias;      // nullable
    const void* state_in;   // (R, K-1), nullable
    void* out;
    void* state_out;        // (R, K-1), nullable
    int64_t Dn, L, R;
};

// Vectorised forward: V = 16 / sizeof(element) steps per thread.  I: the index type, 32-bit
// when the vector count allows (its division is far shorter than a 64-bit one).  RAGGED: rows
// of any length (element-aligned, not whole vectors): element-aligned 16-byte loads and stores,
// the row's last, partial vector element by element (no access leaves the row), and the final
// state left to conv_state_kernel.
template <class E, int K, bool SILU, class I, bool RAGGED>
__device__ __forceinline__ void conv_vec(const ConvArgs& a, I g, I nv) {
    constexpr int V = E::kPerVec;
    const I r = g / nv, q = g % nv;
    const int64_t d = static_cast<int64_t>(r % static_cast<I>(a.Dn));
    const int64_t r64 = static_cast<int64_t>(r), q64 = static_cast<int64_t>(q);
    const auto* xs = static_cast<const typename E::storage*>(a.x) + r64 * a.L;
    const bool whole = !RAGGED || q64 * V + V <= a.L;  // this vector lies inside the row
    uint4 raw;
    if (!RAGGED) {
        raw = *reinterpret_cast<const uint4*>(xs + q64 * V);
    } else if (whole) {
        __builtin_memcpy(&raw, xs + q64 * V, 16);
    } else {
        float f[V];
#pragma unroll
        for (int e = 0; e < V; ++e) f[e] = q64 * V + e < a.L ? E::load1(xs, q64 * V + e) : 0.0f;
        raw = E::pack(f);  // exact: the values came from this storage type
    }
    // the vector before it in the row (a cache hit: the neighbouring lane loads it too; always
    // whole), issued before either is used
    uint4 praw = make_uint4(0, 0, 0, 0);
    if (q > 0) {
        if (RAGGED) __builtin_memcpy(&praw, xs + (q64 - 1) * V, 16);
        else praw = *reinterpret_cast<const uint4*>(xs + (q64 - 1) * V);
    }
    float v[V], pv[V];
    E::unpack(raw, v);
    E::unpack(praw, pv);

    // the K - 1 inputs before this vector, oldest first: the previous vector's tail, or at a row
    // start the carried state (zeros without one)
    float halo[kMaxK - 1];
#pragma unroll
    for (int j = 0; j < K - 1; ++j)
        halo[j] = q > 0 ? pv[V - (K - 1) + j] : (a.state_in ? E::load1(a.state_in, r64 * (K - 1) + j) : 0.0f);
    float wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k] = a.w[d * K + k];
    const float b = a.bias ? a.bias[d] : 0.0f;
    float o[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        float y = b;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int src = e + k - (K - 1);  // index into this vector, negative: the halo
            y = fmaf(wk[k], src >= 0 ? v[src] : halo[src + K - 1], y);
        }
        o[e] = SILU ? silu(y) : y;
    }
    auto* os = static_cast<typename E::storage*>(a.out) + r64 * a.L;
    const uint4 packed = E::pack(o);
    if (!RAGGED) {
        *reinterpret_cast<uint4*>(os + q64 * V) = packed;
    } else if (whole) {
        __builtin_memcpy(os + q64 * V, &packed, 16);
    } else {
#pragma unroll
        for (int e = 0; e < V; ++e)
            if (q64 * V + e < a.L) E::store1(os, q64 * V + e, o[e]);
    }
    if (!RAGGED && a.state_out && q == nv - 1) {
#pragma unroll
        for (int j = 0; j < K - 1; ++j) E::store1(a.state_out, r64 * (K - 1) + j, v[V - (K - 1) + j]);
    }
}

// The grid is capped (a dispatch holds at most 2^32 - 1 work-items per dimension): threads
// stride over the vectors; at the usual sizes each thread takes exactly one.
template <class E, int K, bool SILU, class I, bool RAGGED>
__global__ __launch_bounds__(256) void conv_fwd_vec_kernel(ConvArgs a) {
    constexpr int V = E::kPerVec;
    const I nv = static_cast<I>(RAGGED ? (a.L + V - 1) / V : a.L / V);  // vectors per row
    const I total = static_cast<I>(a.R) * nv;
    const I stride = static_cast<I>(gridDim.x) * static_cast<I>(blockDim.x);
    for (I g = static_cast<I>(blockIdx.x) * static_cast<I>(blockDim.x) + static_cast<I>(threadIdx.x); g < total;
         g += stride)
        conv_vec<E, K, SILU, I, RAGGED>(a, g, nv);
}

// final state for rows of any length (and for L = 0): the last K - 1 inputs,
// taken from the carried state where the sequence is shorter than that.
template <class E, int K>
__global__ __launch_bounds__(256) void conv_state_kernel(ConvArgs a) {
    const int64_t total = a.R * (K - 1);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / (K - 1), j = i % (K - 1);
        const int64_t s = a.L - (K - 1) + j;  // position of state slot j in the sequence
        float v;
        if (s >= 0) v = E::load1(a.x, r * a.L + s);
        else v = a.state_in ? E::load1(a.state_in, r * (K - 1) + (s + K - 1)) : 0.0f;
        E::store1(a.state_out, i, v);
    }
}

// One token per row: the window is the K - 1 kept inputs and x; the kept inputs shift by one.
template <class E, int K, bool SILU>
__global__ __launch_bounds__(256) void conv_update_kernel(void* state, const void* x, const float* w,
                                                          const float* bias, void* out, int64_t R,
                                                          int64_t Dn) {
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < R;
         r += (int64_t)gridDim.x * blockDim.x) {
        const int64_t d = r % Dn;
        float win[K];
#pragma unroll
        for (int j = 0; j < K - 1; ++j) win[j] = E::load1(state, r * (K - 1) + j);
        win[K - 1] = E::load1(x, r);
        float y = bias ? bias[d] : 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) y = fmaf(w[d * K + k], win[k], y);
        E::store1(out, r, SILU ? silu(y) : y);
#pragma unroll
        for (int j = 0; j < K - 1; ++j) E::store1(state, r * (K - 1) + j, win[j + 1]);
    }
}

unsigned blocks_for(int64_t n, int64_t cap = 1 << 20) {
    int64_t b = (n + 255) / 256;
    if (b < 1) b = 1;
    if (b > cap) b = cap;
    return static_cast<unsigned>(b);
}

template <class E, int K, bool SILU, bool RAGGED>
void fwd_vec(const ConvArgs& a, hipStream_t s) {
    constexpr int V = E::kPerVec;
    const int64_t total = a.R * ((a.L + V - 1) / V);
    const dim3 grid(blocks_for(total, 1 << 22));
    if (total + (int64_t{1} << 30) < (int64_t)UINT32_MAX)
        conv_fwd_vec_kernel<E, K, SILU, uint32_t, RAGGED><<<grid, dim3(256), 0, s>>>(a);
    else
        conv_fwd_vec_kernel<E, K, SILU, int64_t, RAGGED><<<grid, dim3(256), 0, s>>>(a);
}

// vec: rows are whole aligned 16-byte vectors; otherwise the element-aligned variant.
template <class E, int K, bool SILU>
hipError_t fwd_t(const ConvArgs& a, bool vec, hipStream_t s) {
    if (a.L > 0) {
        if (vec) fwd_vec<E, K, SILU, false>(a, s);
        else fwd_vec<E, K, SILU, true>(a, s);
    }
    // the aligned vector path writes the final state itself (L >= V >= K - 1 there)
    if (K > 1 && a.state_out && (!vec || a.L == 0))
        conv_state_kernel<E, K><<<dim3(blocks_for(a.R * (K - 1))), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

template <class E, int K>
hipError_t fwd_k(const ConvArgs& a, bool silu_on, bool vec, hipStream_t s) {
    return silu_on ? fwd_t<E, K, true>(a, vec, s) : fwd_t<E, K, false>(a, vec, s);
}

template <class E>
hipError_t fwd_e(const ConvArgs& a, int K, bool silu_on, bool vec, hipStream_t s) {
    switch (K) {
        case 1: return fwd_k<E, 1>(a, silu_on, vec, s);
        case 2: return fwd_k<E, 2>(a, silu_on, vec, s);
        case 3: return fwd_k<E, 3>(a, silu_on, vec, s);
        default: return fwd_k<E, 4>(a, silu_on, vec, s);
    }
}

template <class E, int K>
hipError_t upd_k(const ConvUpdateLaunch& a, hipStream_t s) {
    const unsigned g = blocks_for(a.R);
    if (a.silu) conv_update_kernel<E, K, true><<<dim3(g), dim3(256), 0, s>>>(a.state, a.x, a.w, a.bias, a.out, a.R, a.Dn);
    else conv_update_kernel<E, K, false><<<dim3(g), dim3(256), 0, s>>>(a.state, a.x, a.w, a.bias, a.out, a.R, a.Dn);
    return hipGetLastError();
}

template <class E>
hipError_t upd_e(const ConvUpdateLaunch& a, hipStream_t s) {
    switch (a.K) {
        case 1: return upd_k<E, 1>(a, s);
        case 2: return upd_k<E, 2>(a, s);
        case 3: return upd_k<E, 3>(a, s);
        default: return upd_k<E, 4>(a, s);
    }
}

}  // namespace

hipError_t launch_conv1d_fwd(const ConvLaunch& l, hipStream_t stream) {
    if (l.R == 0) return hipSuccess;
    ConvArgs a;
    a.x = l.x; a.w = l.w; a.bias = l.bias; a.state_in = l.state_in; a.out = l.out;
    a.state_out = l.state_out; a.Dn = l.Dn; a.L = l.L; a.R = l.R;
    return l.bf16 ? fwd_e<BF16>(a, l.K, l.silu, l.vec_ok, stream) : fwd_e<F32>(a, l.K, l.silu, l.vec_ok, stream);
}

hipError_t launch_conv1d_update(const ConvUpdateLaunch& a, hipStream_t stream) {
    if (a.R == 0) return hipSuccess;
    return a.bf16 ? upd_e<BF16>(a, stream) : upd_e<F32>(a, stream);
}

}  // namespace mss
