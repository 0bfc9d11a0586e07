// ssd_scan.hip -- Mamba-2's SSD layer (the upstream README's Mamba-2 block, d_state 64 or 128) as a
// chunked scan on gfx950 matrix cores.
//
// The layer is the selective recurrence with Mamba-2's tied parameters: per batch b and head h
// (P channels), one scalar A[h], one delta per (b, t, h) shared by the head's channels, and B, C
// per (b, t, group) with heads in contiguous blocks of H / G per group:
//     delta_t = softplus(dt_t + dt_bias[h]),   h_t = exp(delta_t A) h_{t-1} + delta_t x_t B_t^T,
//     y_t = h_t C_t + D[h] x_t,   out_t = y_t silu(z_t)        (h_t: P x N, h_0 = 0).
// Unrolled over a chunk of Q = 64 steps starting from the state H entering it, with the running
// sum cs_t of delta inside the chunk:
//     y_t = exp(A cs_t) (C_t H) + sum_{s <= t} (C_t . B_s) exp(A (cs_t - cs_s)) delta_s x_s + D x_t
//     H'  = exp(A cs_{Q-1}) H + sum_s exp(A (cs_{Q-1} - cs_s)) delta_s x_s B_s^T
// -- dense products over the chunk (C H, C B^T, the masked matrix times X, X^T times the scaled
// B), which run as 16 x 16 x 32 bf16 MFMA tiles with fp32 accumulation.  x, B, C, z are bf16 and
// enter the products exactly; the fp32 operands (the masked matrix M, the scaled B and the state
// H) are split into two bf16 terms, hi = bf16(v) and lo = bf16(v - hi), and both are multiplied,
// so each product keeps about 16 mantissa bits (relative error ~2^-17) at twice the bf16 MFMA
// cost.  The exponents are differences of running sums inside one chunk, evaluated directly (a
// ratio exp(A cs_t) / exp(A cs_s) would underflow for long decays).
//
// One workgroup = (b, h, block of 32 of the head's channels), 4 wavefronts, walking the chunks in
// order; H for the block (32 x N fp32) lives in the MFMA accumulators of the wavefronts that
// compute it.  Per chunk: the x / z / B / C tiles are staged in LDS (x and B also transposed, so
// that every MFMA operand is one 16-byte LDS read per lane), the next chunk's tiles are loaded
// into registers meanwhile, and wavefront w computes output rows 16w..16w+15 and a quarter of the
// new state.
#include "device_math.hpp"
#include "mss_internal.hpp"

namespace mss {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kQ = 64;    // chunk length
constexpr int kP = 64;    // channels per head
constexpr int kPB = 32;   // channels per workgroup
constexpr int kPadQ = kQ + 8;  // LDS pitch (elements) of rows indexed by time
constexpr int kThreads = 256;

__device__ __forceinline__ float bf(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }

__device__ __forceinline__ uint16_t to_bf(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }

// hi = bf16(v), lo = bf16(v - hi)
__device__ __forceinline__ void split(float v, uint16_t& hi, uint16_t& lo) {
    hi = to_bf(v);
    lo = to_bf(v - bf(hi));
}

__device__ __forceinline__ f32x4v mfma(const bf16x8& a, const bf16x8& b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The 16-byte MFMA operand of this lane from a matrix stored [row][k] (k contiguous): row
// r0 + lane % 16, k = k0 + 8 (lane / 16) .. + 7.  (A operands take rows as M rows; B operands
// are stored transposed, rows as N columns.)
__device__ __forceinline__ bf16x8 operand(const uint16_t* m, int pitch, int r0, int k0) {
    const int l = threadIdx.x & 63;
    return *reinterpret_cast<const bf16x8*>(m + (r0 + (l & 15)) * pitch + k0 + 8 * (l >> 4));
}

template <int N>
struct Smem {
    static constexpr int kPadN = N + 8;
    uint16_t xt[kPB * kPadQ];        // x^T: [p][s]
    uint16_t zs[kQ * (kPB + 8)];     // z: [t][p]
    uint16_t cs_[kQ * kPadN];        // C: [t][n]
    uint16_t bs[kQ * kPadN];         // B: [s][n]
    uint16_t bt[N * kPadQ];          // B^T: [n][s]
    uint16_t mhi[kQ * kPadQ], mlo[kQ * kPadQ];    // masked matrix M: [t][s], hi / lo
    uint16_t hhi[kPB * kPadN], hlo[kPB * kPadN];  // state H^T: [p][n], hi / lo
    float cum[kQ];                   // running sum of delta inside the chunk
    float dl[kQ];                    // delta
};

// One chunk's global tiles held in registers between their load and their LDS staging.
template <int N>
struct Tiles {
    static constexpr int kBC = kQ * N / 8 / kThreads;  // 16-byte pieces of B (and of C) per thread
    uint4 x, z, b[kBC], c[kBC];
    float dt;
};

struct SsdArgs {
    const uint16_t* x;
    const uint16_t* dt;
    const float* A;
    const uint16_t* B;
    const uint16_t* C;
    const float* D;
    const uint16_t* z;
    const float* bias;
    uint16_t* out;
    float* last_state;
    int64_t L;
    int H, G;
    int softplus;
};

__device__ __forceinline__ uint4 zero_unless(bool ok, uint4 v) {
    return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

// Loads chunk c's tiles (L >= 1).  Rows past L read the last row again and are then zeroed, so
// every load is unconditional and inside the tensors.
template <int N, bool HAS_Z>
__device__ __forceinline__ void load_tiles(Tiles<N>& r, const SsdArgs& a, int64_t b, int h, int g, int pb, int64_t c) {
    const int tid = threadIdx.x;
    const int64_t t0 = c * kQ;
    // x, z: row t = tid / 4, 8 channels (tid % 4) * 8 of the block
    {
        const int t = tid >> 2, q = tid & 3;
        const bool ok = t0 + t < a.L;
        const int64_t tt = ok ? t0 + t : a.L - 1;
        const int64_t off = ((b * a.L + tt) * a.H + h) * kP + pb * kPB + q * 8;
        r.x = zero_unless(ok, *reinterpret_cast<const uint4*>(a.x + off));
        r.z = HAS_Z ? zero_unless(ok, *reinterpret_cast<const uint4*>(a.z + off)) : make_uint4(0, 0, 0, 0);
    }
    // B, C: piece k of thread tid covers row s = (tid + k * 256) / (N / 8), 8 states
#pragma unroll
    for (int k = 0; k < Tiles<N>::kBC; ++k) {
        const int i = tid + k * kThreads;
        const int s = i / (N / 8), q = i % (N / 8);
        const bool ok = t0 + s < a.L;
        const int64_t tt = ok ? t0 + s : a.L - 1;
        const int64_t off = ((b * a.L + tt) * a.G + g) * N + q * 8;
        r.b[k] = zero_unless(ok, *reinterpret_cast<const uint4*>(a.B + off));
        r.c[k] = zero_unless(ok, *reinterpret_cast<const uint4*>(a.C + off));
    }
    // dt: wavefront 0, lane t
    if (tid < kQ) {
        const bool ok = t0 + tid < a.L;
        const int64_t tt = ok ? t0 + tid : a.L - 1;
        const float v = bf(a.dt[(b * a.L + tt) * a.H + h]);
        r.dt = ok ? v : 0.0f;
    }
}

template <int N, bool HAS_Z>
__device__ __forceinline__ void stage_tiles(Smem<N>& sm, const Tiles<N>& r, const SsdArgs& a, float bias, int64_t c) {
    constexpr int PN = Smem<N>::kPadN;
    const int tid = threadIdx.x;
    {
        const int t = tid >> 2, q = tid & 3;
        const uint16_t* xv = reinterpret_cast<const uint16_t*>(&r.x);
#pragma unroll
        for (int j = 0; j < 8; ++j) sm.xt[(q * 8 + j) * kPadQ + t] = xv[j];
        if (HAS_Z) *reinterpret_cast<uint4*>(sm.zs + t * (kPB + 8) + q * 8) = r.z;
    }
#pragma unroll
    for (int k = 0; k < Tiles<N>::kBC; ++k) {
        const int i = tid + k * kThreads;
        const int s = i / (N / 8), q = i % (N / 8);
        *reinterpret_cast<uint4*>(sm.bs + s * PN + q * 8) = r.b[k];
        *reinterpret_cast<uint4*>(sm.cs_ + s * PN + q * 8) = r.c[k];
        const uint16_t* bv = reinterpret_cast<const uint16_t*>(&r.b[k]);
#pragma unroll
        for (int j = 0; j < 8; ++j) sm.bt[(q * 8 + j) * kPadQ + s] = bv[j];
    }
    // delta and its running sum inside the chunk (wavefront 0; steps past L have delta 0)
    if (tid < kQ) {
        const int64_t tt = c * kQ + tid;
        float d = 0.0f;
        if (tt < a.L) {
            const float pre = r.dt + bias;
            d = a.softplus ? softplus(pre) : pre;
        }
        float s = d;
#pragma unroll
        for (int o = 1; o < kQ; o <<= 1) {
            const float v = __shfl_up(s, o, 64);
            if (tid >= o) s += v;
        }
        sm.dl[tid] = d;
        sm.cum[tid] = s;
    }
}

template <int N, bool HAS_Z>
__global__ __launch_bounds__(kThreads) void ssd_chunk_kernel(SsdArgs a) {
    constexpr int PN = Smem<N>::kPadN;
    constexpr int NT = N / 32;  // state n-tiles per wavefront
    __shared__ __align__(16) Smem<N> sm;
    const int pb = blockIdx.x, h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int g = h / (a.H / a.G);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const float A2 = a.A[h] * kLog2e;
    const float Dh = a.D ? a.D[h] : 0.0f;
    const float bias = a.bias ? a.bias[h] : 0.0f;
    const int64_t nchunks = (a.L + kQ - 1) / kQ;

    // the state block this wavefront keeps: p-tile w / 2, n-tiles (w % 2) NT .. + NT - 1
    const int hp0 = 16 * (w >> 1);
    const int hn0 = 16 * NT * (w & 1);
    f32x4v hacc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) hacc[i] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    // H^T starts at zero
    for (int i = threadIdx.x; i < kPB * PN; i += kThreads) sm.hhi[i] = sm.hlo[i] = 0;

    Tiles<N> nxt;
    if (nchunks > 0) load_tiles<N, HAS_Z>(nxt, a, b, h, g, pb, 0);
    for (int64_t c = 0; c < nchunks; ++c) {
        __syncthreads();  // the previous chunk's reads of the staged tiles are done
        stage_tiles<N, HAS_Z>(sm, nxt, a, bias, c);
        __syncthreads();
        if (c + 1 < nchunks) load_tiles<N, HAS_Z>(nxt, a, b, h, g, pb, c + 1);

        // ---- outputs of rows t in [16w, 16w + 16): two 16-channel tiles
        f32x4v y[2] = {f32x4v{0, 0, 0, 0}, f32x4v{0, 0, 0, 0}};
        const int t0 = 16 * w;
        // C H (the state entering the chunk), then scaled per row by exp(A cs_t)
        if (c > 0) {
#pragma unroll
            for (int kk = 0; kk < N / 32; ++kk) {
                const bf16x8 ca = operand(sm.cs_, PN, t0, 32 * kk);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    y[nt] = mfma(ca, operand(sm.hhi, PN, 16 * nt, 32 * kk), y[nt]);
                    y[nt] = mfma(ca, operand(sm.hlo, PN, 16 * nt, 32 * kk), y[nt]);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float e = fast_exp2(A2 * sm.cum[t0 + 4 * (l >> 4) + j]);
                y[0][j] *= e;
                y[1][j] *= e;
            }
        }
        // G = C B^T on the s-tiles 0..w, masked and weighted into M, stored as hi / lo rows
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            f32x4v gt = {0.0f, 0.0f, 0.0f, 0.0f};
            if (st <= w) {
#pragma unroll
                for (int kk = 0; kk < N / 32; ++kk)
                    gt = mfma(operand(sm.cs_, PN, t0, 32 * kk), operand(sm.bs, PN, 16 * st, 32 * kk), gt);
            }
            const int s = 16 * st + (l & 15);
            const float cs_s = sm.cum[s], d_s = sm.dl[s];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = t0 + 4 * (l >> 4) + j;
                float m = 0.0f;
                if (s <= t) m = gt[j] * fast_exp2(A2 * (sm.cum[t] - cs_s)) * d_s;
                uint16_t hi, lo;
                split(m, hi, lo);
                sm.mhi[t * kPadQ + s] = hi;
                sm.mlo[t * kPadQ + s] = lo;
            }
        }
        // M X over s < 16 (w + 1) (a wavefront reads back only the rows it wrote)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (32 * kk < 16 * (w + 1)) {
                const bf16x8 mh = operand(sm.mhi, kPadQ, t0, 32 * kk);
                const bf16x8 ml = operand(sm.mlo, kPadQ, t0, 32 * kk);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const bf16x8 xb = operand(sm.xt, kPadQ, 16 * nt, 32 * kk);
                    y[nt] = mfma(mh, xb, y[nt]);
                    y[nt] = mfma(ml, xb, y[nt]);
                }
            }
        }
        // epilogue: + D x, gate, bf16, store (rows past L are not stored)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int p = 16 * nt + (l & 15);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = t0 + 4 * (l >> 4) + j;
                const int64_t tt = c * kQ + t;
                float v = y[nt][j] + Dh * bf(sm.xt[p * kPadQ + t]);
                if (HAS_Z) v *= silu(bf(sm.zs[t * (kPB + 8) + p]));
                if (tt < a.L) a.out[((b * a.L + tt) * a.H + h) * kP + pb * kPB + p] = to_bf(v);
            }
        }
        __syncthreads();  // every wavefront is done reading H^T (hi / lo) for this chunk

        // ---- the state: H^T <- exp(A cs_end) H^T + X^T (w B), w_s = exp(A (cs_end - cs_s)) delta_s
        const float cend = sm.cum[kQ - 1];
        const float eend = fast_exp2(A2 * cend);
#pragma unroll
        for (int i = 0; i < NT; ++i) hacc[i] *= eend;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const bf16x8 xa = operand(sm.xt, kPadQ, hp0, 32 * kk);
            // this lane's 8 steps s = 32 kk + 8 (l / 16) + j and their weights
            float wv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int s = 32 * kk + 8 * (l >> 4) + j;
                wv[j] = fast_exp2(A2 * (cend - sm.cum[s])) * sm.dl[s];
            }
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const bf16x8 braw = operand(sm.bt, kPadQ, hn0 + 16 * i, 32 * kk);
                bf16x8 bh, bl;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float v = wv[j] * static_cast<float>(braw[j]);
                    const __bf16 hv = static_cast<__bf16>(v);
                    bh[j] = hv;
                    bl[j] = static_cast<__bf16>(v - static_cast<float>(hv));
                }
                hacc[i] = mfma(xa, bh, hacc[i]);
                hacc[i] = mfma(xa, bl, hacc[i]);
            }
        }
        // H^T as hi / lo bf16 for the next chunk's C H: element (p = hp0 + 4 (l / 16) + j,
        // n = hn0 + 16 i + l % 16)
#pragma unroll
        for (int i = 0; i < NT; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int p = hp0 + 4 * (l >> 4) + j, n = hn0 + 16 * i + (l & 15);
                uint16_t hi, lo;
                split(hacc[i][j], hi, lo);
                sm.hhi[p * PN + n] = hi;
                sm.hlo[p * PN + n] = lo;
            }
        }
    }
    if (a.last_state) {
        // last_state[b][h][p][n], p = pb * 32 + hp0 + 4 (l / 16) + j
#pragma unroll
        for (int i = 0; i < NT; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int p = pb * kPB + hp0 + 4 * (l >> 4) + j, n = hn0 + 16 * i + (l & 15);
                a.last_state[((b * a.H + h) * kP + p) * N + n] = hacc[i][j];
            }
        }
    }
}

template <int N, bool HAS_Z>
hipError_t launch_n(const SsdArgs& k, int64_t Bt, hipStream_t stream) {
    const dim3 grid(kP / kPB, static_cast<unsigned>(k.H), static_cast<unsigned>(Bt));
    ssd_chunk_kernel<N, HAS_Z><<<grid, dim3(kThreads), 0, stream>>>(k);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ssd_scan(const SsdLaunch& a, hipStream_t stream) {
    SsdArgs k;
    k.x = static_cast<const uint16_t*>(a.x);
    k.dt = static_cast<const uint16_t*>(a.dt);
    k.A = a.A;
    k.B = static_cast<const uint16_t*>(a.B);
    k.C = static_cast<const uint16_t*>(a.C);
    k.D = a.D;
    k.z = static_cast<const uint16_t*>(a.z);
    k.bias = a.bias;
    k.out = static_cast<uint16_t*>(a.out);
    k.last_state = a.last_state;
    k.L = a.L;
    k.H = static_cast<int>(a.H);
    k.G = static_cast<int>(a.G);
    k.softplus = a.softplus;
    const bool hz = a.z != nullptr;
    if (a.N == 64) return hz ? launch_n<64, true>(k, a.Bt, stream) : launch_n<64, false>(k, a.Bt, stream);
    return hz ? launch_n<128, true>(k, a.Bt, stream) : launch_n<128, false>(k, a.Bt, stream);
}

}  // namespace mss
