// ssd_scan.hip -- Mamba-2's SSD layer (the upstream README's Mamba-2 block, d_state 64 or 128) as a
// chunked scan on gfx950 matrix cores.
//
// The layer is the selective recurrence with Mamba-2's tied parameters: per batch b and head h
// (P = 64 channels), one scalar A[h], one delta per (b, t, h) shared by the head's channels, and
// B, C per (b, t, group) with heads in contiguous blocks of H / G per group:
//     delta_t = softplus(dt_t + dt_bias[h]),   h_t = exp(delta_t A) h_{t-1} + delta_t x_t B_t^T,
//     y_t = h_t C_t + D[h] x_t,   out_t = y_t silu(z_t)        (h_t: P x N, h_0 = 0).
// Unrolled over a chunk of Q = 64 steps entered with the state H, with cs_t the running sum of
// delta inside the chunk and cs_end its total, for every channel p:
//     y_t[p]   = exp(A cs_t) sum_n C_t[n] H[p, n]
//              + sum_{s <= t} (C_t . B_s) exp(A (cs_t - cs_s)) delta_s x_s[p] + D x_t[p]
//     H'[p, n] = exp(A cs_end) H[p, n] + sum_s x_s[p] exp(A (cs_end - cs_s)) delta_s B_s[n]
// -- dense products over the chunk (C H^T, C B^T, the masked matrix M times X, X^T times the
// scaled B) on 16 x 16 x 32 bf16 MFMA tiles with fp32 accumulation.  x, B, C, z are bf16 and enter
// the products exactly; the fp32 operands (M, the scaled B and H) are split into two bf16 terms,
// hi = v truncated to bf16 and lo = (v - hi) truncated, and both are multiplied, so each product
// keeps about 16 mantissa bits (relative error <= 2^-15) at twice the bf16 MFMA cost.
//
// The decay of an entry of M, exp(A (cs_t - cs_s)), is taken as E_t F_s with E_t = exp(A (cs_t -
// c)) and F_s = exp(-A (cs_s - c)) around the chunk's middle running sum c whenever every such
// exponent stays within +-100 (base 2: no overflow or underflow in fp32), else entry by entry.
//
// Parallel decomposition: the chunks of each (b, h) are cut into S segments.  A first kernel runs
// the state products alone over every segment but the last, from H = 0, and leaves the segment's
// local end state and its sum of delta; the main kernel folds the earlier segments' pairs into the
// state entering its segment (H <- exp(A sum delta_k) H + H_k, the associative operator of the S6
// scan's segments) and walks its chunks with outputs.  A workgroup is one (b, h, segment) with
// eight wavefronts: wavefront w computes output rows 16 (w % 4) .. + 15 for channels 32 (w / 4) ..
// + 31, and the state rows 16 (w % 4) .. + 15 for half of the n columns, which stay in its MFMA
// accumulators from chunk to chunk.  Per chunk the x / z / B / C tiles are staged in LDS (x and the
// scaled B also transposed, so that every MFMA operand is one 16-byte LDS read per lane) while the
// next chunk's tiles are loaded into registers.
#include "device_math.hpp"
#include "mss_internal.hpp"

namespace mss {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kQ = 64;          // chunk length
constexpr int kP = 64;          // channels per head
constexpr int kPadQ = kQ + 8;   // LDS pitch (elements) of rows indexed by time
constexpr int kPadP = kP + 8;   // LDS pitch of rows indexed by channel
constexpr int kThreads = 512;   // eight wavefronts
constexpr float kMaxExp2 = 100.0f;

__device__ __forceinline__ float bf(uint32_t v16) { return __uint_as_float(v16 << 16); }

__device__ __forceinline__ f32x4v mfma(const bf16x8& a, const bf16x8& b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The 16-byte MFMA operand of this lane from a matrix stored [row][k] (k contiguous): row
// r0 + lane % 16, k = k0 + 8 (lane / 16) .. + 7.  (A operands: rows are M rows; B operands are
// stored transposed, rows are N columns.)
__device__ __forceinline__ bf16x8 operand(const uint16_t* m, int pitch, int r0, int k0) {
    const int l = threadIdx.x & 63;
    return *reinterpret_cast<const bf16x8*>(m + (r0 + (l & 15)) * pitch + k0 + 8 * (l >> 4));
}

// v as hi + lo bf16 halves (upper 16 bits each): hi = v truncated, lo = (v - hi) truncated.
__device__ __forceinline__ void split16(float v, uint16_t& hi, uint16_t& lo) {
    const uint32_t b = __float_as_uint(v);
    hi = static_cast<uint16_t>(b >> 16);
    lo = static_cast<uint16_t>(__float_as_uint(v - __uint_as_float(b & 0xFFFF0000u)) >> 16);
}

template <int N>
struct Smem {
    static constexpr int kPadN = N + 8;
    uint16_t xt[kP * kPadQ];                     // x^T: [p][s]
    uint16_t zs[kQ * kPadP];                     // z: [t][p]
    uint16_t cs[kQ * kPadN];                     // C: [t][n]
    uint16_t bs[kQ * kPadN];                     // B: [s][n]
    uint16_t bwh[N * kPadQ], bwl[N * kPadQ];     // (w B)^T: [n][s], w_s = exp(A (cs_end - cs_s)) delta_s
    uint16_t mh[kQ * kPadQ], ml[kQ * kPadQ];     // M: [t][s]
    uint16_t hh[kP * kPadN], hl[kP * kPadN];     // H: [p][n] (the state entering the chunk)
    float cum[kQ];   // running sum of delta in the chunk
    float dl[kQ];    // delta
    float E[kQ];     // exp(A (cs_t - c))           (factorized decays)
    float F[kQ];     // exp(-A (cs_s - c)) delta_s
    float Eo[kQ];    // exp(A cs_t): the decay of the entering state
    float eend;      // exp(A cs_end)
    int fact;        // 1: the E F factorization holds for this chunk
};

// The state-only kernel's LDS: x^T, (w B)^T and the chunk's factors.
template <int N>
struct SmemState {
    static constexpr int kPadN = N + 8;
    uint16_t xt[kP * kPadQ];
    uint16_t bwh[N * kPadQ], bwl[N * kPadQ];
    float cum[kQ], dl[kQ], E[kQ], F[kQ], Eo[kQ];
    float eend;
    int fact;
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
    float* seg;       // per (b, h, segment < S - 1): local end state [p][n], then the sum of delta
    int64_t L;
    int H, G, S;
    int64_t nchunks;  // chunks of L
    int softplus;
};

__device__ __forceinline__ uint4 zero_unless(bool ok, uint4 v) {
    return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

// One chunk's global tiles in registers between their load and their LDS staging.  x and B are
// loaded with lane = time row and wavefront w = 8-column slice w (+ 8 k for B at N = 128), so that
// their transposed LDS copies are written by a wavefront at consecutive 2-byte addresses (lanes
// one row apart: no bank conflicts); z and C keep 8 threads per row for row-major copies.
template <int N>
struct Tiles {
    static constexpr int kB = N / 64;                  // 8-state slices of B per wavefront
    static constexpr int kC = kQ * N / 8 / kThreads;   // 16-byte pieces of C per thread
    uint4 x, z, b[kB], c[kC];
    float dt;                                          // dt of row lane (every wavefront)
};

// Chunk c's tiles (L >= 1).  Rows past L re-read the last row and are zeroed, so every load is
// unconditional and inside the tensors.  WITH_OUT: also z and C (the main kernel).  bh_row is
// b L H + h (the flat (b, t = 0, h) row of x and dt), bg_row b L G + g (of B and C).
template <int N, bool HAS_Z, bool WITH_OUT>
__device__ __forceinline__ void load_tiles(Tiles<N>& r, const SsdArgs& a, int64_t bh_row, int64_t bg_row,
                                           int64_t c) {
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int64_t t0 = c * kQ;
    {  // lane = row: x slice w, dt, B slices w + 8 k
        const bool ok = t0 + l < a.L;
        const int64_t tt = ok ? t0 + l : a.L - 1;
        r.x = zero_unless(ok, *reinterpret_cast<const uint4*>(a.x + (bh_row + tt * a.H) * kP + 8 * w));
        const float v = bf(a.dt[bh_row + tt * a.H]);
        r.dt = ok ? v : 0.0f;
#pragma unroll
        for (int k = 0; k < Tiles<N>::kB; ++k)
            r.b[k] = zero_unless(ok, *reinterpret_cast<const uint4*>(a.B + (bg_row + tt * a.G) * N + 8 * (w + 8 * k)));
    }
    if (WITH_OUT) {  // 8 threads per row: z (row tid / 8), C pieces
        if (HAS_Z) {
            const int t = tid >> 3, q = tid & 7;
            const bool ok = t0 + t < a.L;
            const int64_t tt = ok ? t0 + t : a.L - 1;
            r.z = zero_unless(ok, *reinterpret_cast<const uint4*>(a.z + (bh_row + tt * a.H) * kP + q * 8));
        }
#pragma unroll
        for (int k = 0; k < Tiles<N>::kC; ++k) {
            const int i = tid + k * kThreads;
            const int s = i / (N / 8), q = i % (N / 8);
            const bool ok = t0 + s < a.L;
            const int64_t tt = ok ? t0 + s : a.L - 1;
            r.c[k] = zero_unless(ok, *reinterpret_cast<const uint4*>(a.C + (bg_row + tt * a.G) * N + q * 8));
        }
    }
}

// Stages chunk c's tiles in LDS.  Every wavefront forms delta and its running sum for the 64 rows
// (lane t), so that it can scale its B slices by w_t = exp(A (cs_end - cs_t)) delta_t and write
// (w B)^T directly; wavefront 0 also publishes the per-row factors.
template <int N, bool HAS_Z, bool WITH_OUT, class SM>
__device__ __forceinline__ void stage_tiles(SM& sm, const Tiles<N>& r, const SsdArgs& a, float A2, float bias,
                                            int64_t c) {
    constexpr int PN = N + 8;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    float d = 0.0f;
    if (c * kQ + l < a.L) {
        const float pre = r.dt + bias;
        d = a.softplus ? softplus(pre) : pre;
    }
    float cum = d;
#pragma unroll
    for (int o = 1; o < kQ; o <<= 1) {
        const float v = __shfl_up(cum, o, 64);
        if (l >= o) cum += v;
    }
    const float cend = __shfl(cum, kQ - 1, 64);
    const float wt = fast_exp2(A2 * (cend - cum)) * d;
    {  // x^T slice w: element (p = 8 w + j, s = l)
        const uint32_t xw[4] = {r.x.x, r.x.y, r.x.z, r.x.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sm.xt[(8 * w + 2 * j) * kPadQ + l] = static_cast<uint16_t>(xw[j]);
            sm.xt[(8 * w + 2 * j + 1) * kPadQ + l] = static_cast<uint16_t>(xw[j] >> 16);
        }
    }
#pragma unroll
    for (int k = 0; k < Tiles<N>::kB; ++k) {  // B row l, states 8 (w + 8 k) .. + 7
        const int n0 = 8 * (w + 8 * k);
        if constexpr (WITH_OUT) *reinterpret_cast<uint4*>(sm.bs + l * PN + n0) = r.b[k];
        const uint32_t bw[4] = {r.b[k].x, r.b[k].y, r.b[k].z, r.b[k].w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint16_t hi, lo;
            split16(wt * bf((bw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu), hi, lo);
            sm.bwh[(n0 + j) * kPadQ + l] = hi;
            sm.bwl[(n0 + j) * kPadQ + l] = lo;
        }
    }
    if constexpr (WITH_OUT) {
        if (HAS_Z) *reinterpret_cast<uint4*>(sm.zs + (tid >> 3) * kPadP + (tid & 7) * 8) = r.z;
#pragma unroll
        for (int k = 0; k < Tiles<N>::kC; ++k) {
            const int i = tid + k * kThreads;
            *reinterpret_cast<uint4*>(sm.cs + (i / (N / 8)) * PN + (i % (N / 8)) * 8) = r.c[k];
        }
    }
    if (w == 0) {
        const float cmid = __shfl(cum, kQ / 2 - 1, 64);
        const float eu = A2 * (cum - cmid);
        const bool all_ok = __all(fabsf(eu) <= kMaxExp2);
        sm.dl[l] = d;
        sm.cum[l] = cum;
        sm.E[l] = fast_exp2(eu);
        sm.F[l] = fast_exp2(-eu) * d;
        sm.Eo[l] = fast_exp2(A2 * cum);
        if (l == 0) {
            sm.eend = fast_exp2(A2 * cend);
            sm.fact = all_ok ? 1 : 0;
        }
    }
}

// H <- exp(A cs_end) H + X^T (w B) for this wavefront's state block (rows p0 .. p0 + 15, columns
// n0 + 16 i), then (PUBLISH) its bf16 halves into hh / hl for the next chunk's products.
template <int N, bool PUBLISH, class SM>
__device__ __forceinline__ void state_step(SM& sm, f32x4v (&hacc)[N / 32], int p0, int n0) {
    constexpr int PN = N + 8;
    const float e = sm.eend;
#pragma unroll
    for (int i = 0; i < N / 32; ++i) hacc[i] *= e;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 xa = operand(sm.xt, kPadQ, p0, 32 * kk);
#pragma unroll
        for (int i = 0; i < N / 32; ++i) {
            hacc[i] = mfma(xa, operand(sm.bwh, kPadQ, n0 + 16 * i, 32 * kk), hacc[i]);
            hacc[i] = mfma(xa, operand(sm.bwl, kPadQ, n0 + 16 * i, 32 * kk), hacc[i]);
        }
    }
    if constexpr (PUBLISH) {
        const int l = threadIdx.x & 63;
#pragma unroll
        for (int i = 0; i < N / 32; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int p = p0 + 4 * (l >> 4) + j, n = n0 + 16 * i + (l & 15);
                uint16_t hi, lo;
                split16(hacc[i][j], hi, lo);
                sm.hh[p * PN + n] = hi;
                sm.hl[p * PN + n] = lo;
            }
        }
    }
}

// Segment `seg` (< S - 1) of (b, h): the state products alone, from H = 0; leaves the local end
// state and the sum of delta.
template <int N>
__global__ __launch_bounds__(kThreads) void ssd_state_kernel(SsdArgs a) {
    __shared__ __align__(16) SmemState<N> sm;
    const int seg = blockIdx.x, h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int g = h / (a.H / a.G);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const float A2 = a.A[h] * kLog2e;
    const float bias = a.bias ? a.bias[h] : 0.0f;
    const int64_t c0 = seg * a.nchunks / a.S, c1 = (seg + 1) * a.nchunks / a.S;
    const int p0 = 16 * (w & 3), n0 = (N / 2) * (w >> 2);
    const int64_t bh_row = b * a.L * a.H + h, bg_row = b * a.L * a.G + g;
    f32x4v hacc[N / 32];
#pragma unroll
    for (int i = 0; i < N / 32; ++i) hacc[i] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    float dsum = 0.0f;
    Tiles<N> nxt;
    if (c0 < c1) load_tiles<N, false, false>(nxt, a, bh_row, bg_row, c0);
    for (int64_t c = c0; c < c1; ++c) {
        __syncthreads();  // the previous chunk's reads of the staged tiles are done
        stage_tiles<N, false, false>(sm, nxt, a, A2, bias, c);
        __syncthreads();
        if (c + 1 < c1) load_tiles<N, false, false>(nxt, a, bh_row, bg_row, c + 1);
        dsum += sm.cum[kQ - 1];
        state_step<N, false>(sm, hacc, p0, n0);
    }
    float* dst = a.seg + ((b * a.H + h) * (a.S - 1) + seg) * (kP * N + 1);
#pragma unroll
    for (int i = 0; i < N / 32; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[(p0 + 4 * (l >> 4) + j) * N + n0 + 16 * i + (l & 15)] = hacc[i][j];
    if (threadIdx.x == 0) dst[kP * N] = dsum;
}

template <int N, bool HAS_Z>
__global__ __launch_bounds__(kThreads) void ssd_main_kernel(SsdArgs a) {
    constexpr int PN = Smem<N>::kPadN;
    __shared__ __align__(16) Smem<N> sm;
    const int seg = blockIdx.x, h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int g = h / (a.H / a.G);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const float A2 = a.A[h] * kLog2e;
    const float Dh = a.D ? a.D[h] : 0.0f;
    const float bias = a.bias ? a.bias[h] : 0.0f;
    const int64_t c0 = seg * a.nchunks / a.S, c1 = (seg + 1) * a.nchunks / a.S;
    const int rt = w & 3;           // row tile: outputs t (and state rows p) 16 rt .. + 15
    const int ct = 2 * (w >> 2);    // output channel tiles ct, ct + 1
    const int p0 = 16 * rt, n0 = (N / 2) * (w >> 2);
    const int64_t bh_row = b * a.L * a.H + h, bg_row = b * a.L * a.G + g;

    // the state entering the segment: the earlier segments' local end states folded in order
    f32x4v hacc[N / 32];
#pragma unroll
    for (int i = 0; i < N / 32; ++i) hacc[i] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = 0; k < seg; ++k) {
        const float* src = a.seg + ((b * a.H + h) * (a.S - 1) + k) * (kP * N + 1);
        const float e = fast_exp2(A2 * src[kP * N]);
#pragma unroll
        for (int i = 0; i < N / 32; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                hacc[i][j] = fmaf(e, hacc[i][j], src[(p0 + 4 * (l >> 4) + j) * N + n0 + 16 * i + (l & 15)]);
    }
#pragma unroll
    for (int i = 0; i < N / 32; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint16_t hi, lo;
            split16(hacc[i][j], hi, lo);
            const int p = p0 + 4 * (l >> 4) + j, n = n0 + 16 * i + (l & 15);
            sm.hh[p * PN + n] = hi;
            sm.hl[p * PN + n] = lo;
        }
    }

    Tiles<N> nxt;
    if (c0 < c1) load_tiles<N, HAS_Z, true>(nxt, a, bh_row, bg_row, c0);
    for (int64_t c = c0; c < c1; ++c) {
        __syncthreads();  // the previous chunk's reads of the staged tiles are done
        stage_tiles<N, HAS_Z, true>(sm, nxt, a, A2, bias, c);
        __syncthreads();
        if (c + 1 < c1) load_tiles<N, HAS_Z, true>(nxt, a, bh_row, bg_row, c + 1);

        const int t0 = 16 * rt;
        const bool fact = sm.fact != 0;
        // outputs of rows t0 .. t0 + 15, channel tiles ct, ct + 1: first the entering state's part
        f32x4v y[2] = {f32x4v{0, 0, 0, 0}, f32x4v{0, 0, 0, 0}};
        if (c > 0) {
#pragma unroll
            for (int kk = 0; kk < N / 32; ++kk) {
                const bf16x8 ca = operand(sm.cs, PN, t0, 32 * kk);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    y[u] = mfma(ca, operand(sm.hh, PN, 16 * (ct + u), 32 * kk), y[u]);
                    y[u] = mfma(ca, operand(sm.hl, PN, 16 * (ct + u), 32 * kk), y[u]);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float e = sm.Eo[t0 + 4 * (l >> 4) + j];
                y[0][j] *= e;
                y[1][j] *= e;
            }
        }
        // M rows t0 .. t0 + 15: this wavefront takes s-tiles w / 4 and w / 4 + 2 (the other
        // wavefront of the row tile the other two); tiles past the diagonal are zeros
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const int st = (w >> 2) + 2 * v;
            f32x4v gt = {0.0f, 0.0f, 0.0f, 0.0f};
            if (st <= rt) {
#pragma unroll
                for (int kk = 0; kk < N / 32; ++kk)
                    gt = mfma(operand(sm.cs, PN, t0, 32 * kk), operand(sm.bs, PN, 16 * st, 32 * kk), gt);
            }
            const int s = 16 * st + (l & 15);
            const float Fs = sm.F[s], cs_s = sm.cum[s], d_s = sm.dl[s];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = t0 + 4 * (l >> 4) + j;
                const float dec = fact ? sm.E[t] * Fs : fast_exp2(A2 * (sm.cum[t] - cs_s)) * d_s;
                const float m = s <= t ? gt[j] * dec : 0.0f;
                uint16_t hi, lo;
                split16(m, hi, lo);
                sm.mh[t * kPadQ + s] = hi;
                sm.ml[t * kPadQ + s] = lo;
            }
        }
        __syncthreads();  // M rows complete; every read of the entering H done
        // + M X over s < 16 (rt + 1)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (32 * kk < 16 * (rt + 1)) {
                const bf16x8 mh = operand(sm.mh, kPadQ, t0, 32 * kk);
                const bf16x8 ml = operand(sm.ml, kPadQ, t0, 32 * kk);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const bf16x8 xb = operand(sm.xt, kPadQ, 16 * (ct + u), 32 * kk);
                    y[u] = mfma(mh, xb, y[u]);
                    y[u] = mfma(ml, xb, y[u]);
                }
            }
        }
        // + D x, gate, bf16 (round to nearest even), store; rows past L are not stored
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int p = 16 * (ct + u) + (l & 15);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = t0 + 4 * (l >> 4) + j;
                float v = y[u][j] + Dh * bf(sm.xt[p * kPadQ + t]);
                if (HAS_Z) v *= silu(bf(sm.zs[t * kPadP + p]));
                if (c * kQ + t < a.L)
                    a.out[(bh_row + (c * kQ + t) * a.H) * kP + p] =
                        __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
            }
        }
        // the state for the next chunk (H is read again only after the next chunk's barriers)
        state_step<N, true>(sm, hacc, p0, n0);
    }
    if (a.last_state && seg == a.S - 1) {
        float* dst = a.last_state + (b * a.H + h) * kP * N;
#pragma unroll
        for (int i = 0; i < N / 32; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[(p0 + 4 * (l >> 4) + j) * N + n0 + 16 * i + (l & 15)] = hacc[i][j];
    }
}

template <int N, bool HAS_Z>
hipError_t launch_n(const SsdArgs& k, int64_t Bt, hipStream_t stream) {
    const dim3 block(kThreads);
    if (k.S > 1)
        ssd_state_kernel<N><<<dim3(static_cast<unsigned>(k.S - 1), static_cast<unsigned>(k.H),
                                   static_cast<unsigned>(Bt)), block, 0, stream>>>(k);
    ssd_main_kernel<N, HAS_Z><<<dim3(static_cast<unsigned>(k.S), static_cast<unsigned>(k.H),
                                     static_cast<unsigned>(Bt)), block, 0, stream>>>(k);
    return hipGetLastError();
}

}  // namespace

// Segments per (batch, head): about four rounds of workgroups for the chip (the LDS holds one
// workgroup per CU), at least two chunks each.
int plan_ssd_segments(const SsdLaunch& a, int num_cus, int segments_override) {
    const int64_t nchunks = (a.L + kQ - 1) / kQ;
    const int64_t pairs = a.Bt * a.H;
    const int64_t target = 4LL * (num_cus > 0 ? num_cus : 256);
    int64_t S = pairs > 0 ? (target + pairs - 1) / pairs : 1;
    if (S > nchunks / 2) S = nchunks / 2;
    if (segments_override > 0) S = segments_override;
    if (S > nchunks) S = nchunks;
    if (S > 65535) S = 65535;
    if (S < 1) S = 1;
    return static_cast<int>(S);
}

size_t ssd_workspace_bytes(const SsdLaunch& a, int segments) {
    return segments > 1 ? static_cast<size_t>(a.Bt * a.H) * (segments - 1) * (kP * a.N + 1) * sizeof(float) : 0;
}

hipError_t launch_ssd_scan(const SsdLaunch& a, int segments, float* workspace, hipStream_t stream) {
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
    k.seg = workspace;
    k.L = a.L;
    k.H = static_cast<int>(a.H);
    k.G = static_cast<int>(a.G);
    k.S = segments;
    k.nchunks = (a.L + kQ - 1) / kQ;
    k.softplus = a.softplus;
    const bool hz = a.z != nullptr;
    if (a.N == 64) return hz ? launch_n<64, true>(k, a.Bt, stream) : launch_n<64, false>(k, a.Bt, stream);
    return hz ? launch_n<128, true>(k, a.Bt, stream) : launch_n<128, false>(k, a.Bt, stream);
}

}  // namespace mss
