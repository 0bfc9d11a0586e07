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
//              + sum_{s <= t} (B_s . C_t) exp(A (cs_t - cs_s)) delta_s x_s[p] + D x_t[p]
//     H'[p, n] = exp(A cs_end) H[p, n] + sum_s B_s[n] w_s x_s[p],   w_s = exp(A (cs_end - cs_s)) delta_s
// -- dense products over the chunk on 16 x 16 x 32 bf16 MFMA tiles with fp32 accumulation.  x, B,
// C, z are bf16 and enter the products exactly; fp32 operands (the masked decay matrix, the state,
// w x) are split into two bf16 terms, hi = bf16(v) and lo = bf16(v - hi) (round to nearest), and both
// are multiplied: each product keeps about 17 mantissa bits.
//
// Everything is computed transposed, output rows indexed by channel: Y^T[p][t] and the state as
// H^T[n][p].  In an MFMA result a lane holds four consecutive rows of one column, so
//   * a lane's outputs are four consecutive channels of one time step (8-byte stores; x and z are
//     loaded in that layout and never staged);
//   * the masked decay matrix M^T[s][t] = (B_s . C_t) exp(A (cs_t - cs_s)) delta_s comes out of its
//     MFMA (A operand B, B operand C, contracted over n) with four consecutive s per lane, and the
//     contraction of Y^T = X^T M^T over s can take two such tiles as its B operand directly, with
//     the 32 k-slots of the instruction assigned to s in that order (the A operand, x^T, is read
//     with the same assignment).  The state H^T feeds the C H product the same way.  Neither M nor
//     H passes through LDS.
// The decay of an entry of M is taken as E_t F_s with E_t = exp(A (cs_t - c)) and F_s = exp(-A
// (cs_s - c)) delta_s around the chunk's middle running sum c whenever every such exponent stays
// within +-100 (base 2: no overflow or underflow in fp32); E_t then scales the finished Y^T column.
// Otherwise the entries take their own exponentials.
//
// Parallel decomposition: the chunks of each (b, h) are cut into S segments.  A first kernel runs
// the state products alone over every segment but the last, from H = 0, and leaves the segment's
// local end state and its sum of delta; the main kernel folds the earlier segments' pairs into the
// state entering its segment (H <- exp(A sum delta_k) H + H_k, the associative operator of the S6
// scan's segments) and walks its chunks with outputs.  A workgroup is one (b, h, segment) with four
// wavefronts; wavefront w owns channels 16 w .. 16 w + 15: their state columns (in MFMA
// accumulators from chunk to chunk) and all 64 x 16 outputs of a chunk.  The B . C products and the
// decays are formed by each wavefront for itself; B, C, B^T and x^T of the chunk are staged in LDS
// (B^T and x^T written transposed by lanes one time step apart: no bank conflicts), while the next
// chunk's tiles are loaded into registers.
#include "device_math.hpp"
#include "mss_internal.hpp"

namespace mss {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQ = 64;          // chunk length
constexpr int kP = 64;          // channels per head
constexpr int kPadQ = kQ + 8;   // LDS pitch (elements) of rows indexed by time
constexpr int kThreads = 256;   // four wavefronts
constexpr float kMaxExp2 = 100.0f;

__device__ __forceinline__ float bf(uint32_t v16) { return __uint_as_float(v16 << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ f32x4v mfma(const bf16x8& a, const bf16x8& b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_op(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// a, b rounded to bf16 (nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){a, b}, bf16x2));
}

// The hi / lo bf16 terms of the pair (a, b), each packed as pack2 packs them: {hi, lo}.
__device__ __forceinline__ u32x2 split2(float a, float b) {
    const uint32_t hi = pack2(a, b);
    return u32x2{hi, pack2(a - bf_lo(hi), b - bf_hi(hi))};
}

// The hi and lo bf16x8 operands of the pairs (v0, v1), (v2, v3), (v4, v5), (v6, v7).
__device__ __forceinline__ void split8(float v0, float v1, float v2, float v3, float v4, float v5, float v6,
                                       float v7, bf16x8& hi, bf16x8& lo) {
    const u32x2 a = split2(v0, v1), b = split2(v2, v3), c = split2(v4, v5), d = split2(v6, v7);
    hi = as_op(u32x4{a[0], b[0], c[0], d[0]});
    lo = as_op(u32x4{a[1], b[1], c[1], d[1]});
}

// The 16-byte MFMA operand of this lane from a matrix stored [row][k] (k contiguous): row
// r0 + lane % 16, k = k0 + 8 (lane / 16) .. + 7.
__device__ __forceinline__ bf16x8 operand(const uint16_t* m, int pitch, int r0, int k0) {
    const int l = threadIdx.x & 63;
    return *reinterpret_cast<const bf16x8*>(m + (r0 + (l & 15)) * pitch + k0 + 8 * (l >> 4));
}

// The same row's operand with the k-slots of the permuted assignment: slots 8 (lane / 16) .. + 3
// hold k = k0 + 4 (lane / 16) .. + 3 and slots 8 (lane / 16) + 4 .. + 7 hold k = k0 + 16 + 4 (lane
// / 16) .. + 3 -- the order in which an MFMA result tile pair (rows k0 .., k0 + 16 ..) holds them.
__device__ __forceinline__ bf16x8 operand_perm(const uint16_t* m, int pitch, int r0, int k0) {
    const int l = threadIdx.x & 63;
    const uint16_t* row = m + (r0 + (l & 15)) * pitch + k0 + 4 * (l >> 4);
    const u32x2 a = *reinterpret_cast<const u32x2*>(row);
    const u32x2 b = *reinterpret_cast<const u32x2*>(row + 16);
    return as_op(u32x4{a[0], a[1], b[0], b[1]});
}

// Inclusive prefix sum over the 64 lanes: shifts within rows of 16, then the row carries.
__device__ __forceinline__ float wave_prefix_sum(float v) {
    int x = __float_as_int(v);
    x = __float_as_int(__int_as_float(x) + __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true)));
    x = __float_as_int(__int_as_float(x) + __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true)));
    x = __float_as_int(__int_as_float(x) + __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true)));
    x = __float_as_int(__int_as_float(x) + __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true)));
    // row_bcast:15 into rows 1 and 3, then row_bcast:31 into rows 2 and 3
    x = __float_as_int(__int_as_float(x) + __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false)));
    x = __float_as_int(__int_as_float(x) + __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false)));
    return __int_as_float(x);
}

__device__ __forceinline__ float lane_value(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// LDS of a workgroup.  OUT (the main kernel): also B and C row-major and the output decays.
template <int N, bool OUT>
struct Smem {
    static constexpr int kPadN = N + 8;
    static constexpr int kRowMajor = OUT ? kQ * kPadN : 8;
    uint16_t xt[kP * kPadQ];        // x^T [p][s]
    uint16_t bt[N * kPadQ];         // B^T [n][s]
    uint16_t bs[kRowMajor];         // B [s][n]
    uint16_t cs[kRowMajor];         // C [t][n]
    float w[kQ];                    // exp(A (cs_end - cs_s)) delta_s
    float F[kQ];                    // exp(-A (cs_s - c)) delta_s   (factorized decays)
    float E[kQ];                    // exp(A (cs_t - c))
    float Eo[kQ];                   // exp(A cs_t): the decay of the entering state
    float cum[kQ];                  // running sum of delta
    float dl[kQ];                   // delta
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
    float* seg;       // per (b, h, segment < S - 1): local end state (accumulator order), then sum of delta
    int64_t L;
    int H, G, S;
    int64_t nchunks;  // chunks of L
    int softplus;
};

// One chunk's global tiles in registers between their load and their LDS staging.  x: four time
// rows t = 16 i + lane % 16, channels 16 w + 4 (lane / 16) .. + 3 (the output layout); dt, B and C:
// time row lane, 8-state slices w + 4 k.  Rows past L hold copies of row L - 1 (finite values):
// their delta is set to 0 at staging, which zeroes their weight in every product that reaches a
// stored output or the state, and their outputs are not stored.  (The loads are used as they
// arrive, with no select on them, so that nothing waits for them before the staging.)
template <int N>
struct Tiles {
    static constexpr int kS = N / 32;  // slices of B (and C) per wavefront
    u32x2 x[4];
    u32x4 b[kS], c[kS];
    uint16_t dt;
};

// A 64-step row block in the output layout (x or z); rows past L read row L - 1.
__device__ __forceinline__ void load_rows4(u32x2 (&r)[4], const uint16_t* base, const SsdArgs& a, int64_t bh_row,
                                           int64_t t0) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + 16 * i + (l & 15);
        const int64_t tc = t < a.L ? t : a.L - 1;
        r[i] = *reinterpret_cast<const u32x2*>(base + (bh_row + tc * a.H) * kP + 16 * w + 4 * (l >> 4));
    }
}

// Chunk c's tiles (L >= 1).  Every load is unconditional and inside the tensors.  bh_row is
// b L H + h (the flat (b, t = 0, h) row of x and dt), bg_row b L G + g (of B and C).
template <int N, bool OUT>
__device__ __forceinline__ void load_tiles(Tiles<N>& r, const SsdArgs& a, int64_t bh_row, int64_t bg_row,
                                           int64_t c) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int64_t t0 = c * kQ;
    load_rows4(r.x, a.x, a, bh_row, t0);
    const int64_t tc = t0 + l < a.L ? t0 + l : a.L - 1;
    r.dt = a.dt[bh_row + tc * a.H];
#pragma unroll
    for (int k = 0; k < Tiles<N>::kS; ++k) {
        const int n0 = 8 * (w + 4 * k);
        r.b[k] = *reinterpret_cast<const u32x4*>(a.B + (bg_row + tc * a.G) * N + n0);
        if (OUT) r.c[k] = *reinterpret_cast<const u32x4*>(a.C + (bg_row + tc * a.G) * N + n0);
    }
}

struct ChunkInfo {
    float eend;  // exp(A cs_end)
    float cend;  // cs_end
    bool fact;   // the E F factorization holds
};

// Stages chunk c's tiles in LDS.  Every wavefront forms delta and its running sum for the 64 rows
// (lane t) itself, so the chunk's scalars are uniform without a round trip; wavefront 0 publishes
// the per-row factors.
template <int N, bool OUT>
__device__ __forceinline__ ChunkInfo stage_tiles(Smem<N, OUT>& sm, const Tiles<N>& r, const SsdArgs& a, float A2,
                                                 float bias, int64_t c) {
    constexpr int PN = Smem<N, OUT>::kPadN;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    float d = 0.0f;
    if (c * kQ + l < a.L) {
        const float pre = bf(r.dt) + bias;
        d = a.softplus ? softplus(pre) : pre;
    }
    const float cum = wave_prefix_sum(d);
    ChunkInfo ci;
    ci.cend = lane_value(cum, kQ - 1);
    ci.eend = fast_exp2(A2 * ci.cend);
    const float cmid = lane_value(cum, kQ / 2 - 1);
    const float eu = A2 * (cum - cmid);
    ci.fact = __all(fabsf(eu) <= kMaxExp2);
    if (w == 0) {
        sm.w[l] = fast_exp2(A2 * (ci.cend - cum)) * d;
        if (OUT) {
            sm.F[l] = fast_exp2(-eu) * d;
            sm.E[l] = fast_exp2(eu);
            sm.Eo[l] = fast_exp2(A2 * cum);
            sm.cum[l] = cum;
            sm.dl[l] = d;
        }
    }
    // x^T rows 16 w + 4 (l / 16) + j, columns 16 i + l % 16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint16_t* dst = sm.xt + (16 * w + 4 * (l >> 4)) * kPadQ + 16 * i + (l & 15);
        dst[0] = static_cast<uint16_t>(r.x[i][0]);
        dst[kPadQ] = static_cast<uint16_t>(r.x[i][0] >> 16);
        dst[2 * kPadQ] = static_cast<uint16_t>(r.x[i][1]);
        dst[3 * kPadQ] = static_cast<uint16_t>(r.x[i][1] >> 16);
    }
    // B^T columns l (and B, C rows l)
#pragma unroll
    for (int k = 0; k < Tiles<N>::kS; ++k) {
        const int n0 = 8 * (w + 4 * k);
#pragma unroll
        for (int j = 0; j < 8; ++j) sm.bt[(n0 + j) * kPadQ + l] = static_cast<uint16_t>(r.b[k][j >> 1] >> (16 * (j & 1)));
        if (OUT) {
            *reinterpret_cast<u32x4*>(sm.bs + l * PN + n0) = r.b[k];
            *reinterpret_cast<u32x4*>(sm.cs + l * PN + n0) = r.c[k];
        }
    }
    return ci;
}

// H^T <- exp(A cs_end) H^T + B^T (w x) for this wavefront's channels: hacc[i] is the tile of states
// 16 i .. + 15 (rows) by channels 16 w .. + 15 (columns).
template <int N, bool OUT>
__device__ __forceinline__ void state_step(const Smem<N, OUT>& sm, f32x4v (&hacc)[N / 16], float eend) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < N / 16; ++i) hacc[i] *= eend;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        // B operand (k = s, column p): w_s x_s[p] for s = 32 kk + 8 (l / 16) .. + 7
        const int s0 = 32 * kk + 8 * (l >> 4);
        const u32x4 xv = *reinterpret_cast<const u32x4*>(sm.xt + (16 * w + (l & 15)) * kPadQ + s0);
        const f32x4v w0 = *reinterpret_cast<const f32x4v*>(sm.w + s0);
        const f32x4v w1 = *reinterpret_cast<const f32x4v*>(sm.w + s0 + 4);
        bf16x8 xh, xl;
        split8(bf_lo(xv[0]) * w0[0], bf_hi(xv[0]) * w0[1], bf_lo(xv[1]) * w0[2], bf_hi(xv[1]) * w0[3],
               bf_lo(xv[2]) * w1[0], bf_hi(xv[2]) * w1[1], bf_lo(xv[3]) * w1[2], bf_hi(xv[3]) * w1[3], xh, xl);
#pragma unroll
        for (int i = 0; i < N / 16; ++i) {
            const bf16x8 bo = operand(sm.bt, kPadQ, 16 * i, 32 * kk);
            hacc[i] = mfma(bo, xh, hacc[i]);
            hacc[i] = mfma(bo, xl, hacc[i]);
        }
    }
}

// Where segment k of (b, h) keeps its local end state: the accumulators of wavefront w in order
// (tile i, element j, lane), so the stores and loads of a wavefront are 256-byte runs.
__device__ __forceinline__ float* seg_slot(const SsdArgs& a, int64_t b, int h, int k, int n_states) {
    return a.seg + ((b * a.H + h) * (a.S - 1) + k) * (static_cast<int64_t>(kP) * n_states + 1);
}

// Segment `seg` (< S - 1) of (b, h): the state products alone, from H = 0; leaves the local end
// state and the sum of delta.
template <int N>
__global__ __launch_bounds__(kThreads) void ssd_state_kernel(SsdArgs a) {
    __shared__ __align__(16) Smem<N, false> sm;
    const int seg = blockIdx.x, h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int g = h / (a.H / a.G);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const float A2 = a.A[h] * kLog2e;
    const float bias = a.bias ? a.bias[h] : 0.0f;
    const int64_t c0 = seg * a.nchunks / a.S, c1 = (seg + 1) * a.nchunks / a.S;
    const int64_t bh_row = b * a.L * a.H + h, bg_row = b * a.L * a.G + g;
    f32x4v hacc[N / 16];
#pragma unroll
    for (int i = 0; i < N / 16; ++i) hacc[i] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    float dsum = 0.0f;
    Tiles<N> nxt;
    if (c0 < c1) load_tiles<N, false>(nxt, a, bh_row, bg_row, c0);
    for (int64_t c = c0; c < c1; ++c) {
        __syncthreads();  // the previous chunk's reads of the staged tiles are done
        const ChunkInfo ci = stage_tiles<N, false>(sm, nxt, a, A2, bias, c);
        __syncthreads();
        load_tiles<N, false>(nxt, a, bh_row, bg_row, c + 1 < c1 ? c + 1 : c);  // unconditional (see below)
        dsum += ci.cend;
        state_step<N, false>(sm, hacc, ci.eend);
    }
    float* dst = seg_slot(a, b, h, seg, N) + w * (N / 16) * 4 * 64 + l;
#pragma unroll
    for (int i = 0; i < N / 16; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[(4 * i + j) * 64] = hacc[i][j];
    if (threadIdx.x == 0) seg_slot(a, b, h, seg, N)[kP * N] = dsum;
}

// The chunk's outputs for this wavefront's channels, t-tile by t-tile: Y^T = E_t (X^T M^T) +
// Eo_t (H C^T) + D x, gated and stored.  FAST: the decays factorize and all 64 rows are inside L
// (straight-line code); otherwise the entries of M take their own exponentials when the chunk
// needs them and rows at or past `valid` are not stored.
template <int N, bool HAS_Z, bool FAST>
__device__ __forceinline__ void chunk_outputs(const Smem<N, true>& sm, const ChunkInfo& ci,
                                              const f32x4v (&hacc)[N / 16], const u32x2 (&zc)[4], float A2,
                                              float Dh, uint16_t* orow, int H, int64_t valid) {
    constexpr int PN = Smem<N, true>::kPadN;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const bool fact = FAST || ci.fact;
    // H C^T for the four t-tiles first: the entering state as the A operand (rows p, k = n in the
    // permuted order), one 32-state block at a time
    f32x4v yo[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) yo[tt] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < N / 32; ++k) {
        bf16x8 hh, hl;
        split8(hacc[2 * k][0], hacc[2 * k][1], hacc[2 * k][2], hacc[2 * k][3], hacc[2 * k + 1][0],
               hacc[2 * k + 1][1], hacc[2 * k + 1][2], hacc[2 * k + 1][3], hh, hl);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const bf16x8 co = operand_perm(sm.cs, PN, 16 * tt, 32 * k);
            yo[tt] = mfma(hh, co, yo[tt]);
            yo[tt] = mfma(hl, co, yo[tt]);
        }
    }
    // x^T operands of this wavefront's channels, permuted k = s order
    const bf16x8 xo0 = operand_perm(sm.xt, kPadQ, 16 * w, 0);
    const bf16x8 xo1 = operand_perm(sm.xt, kPadQ, 16 * w, 32);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int t = 16 * tt + (l & 15);  // this lane's output time step in the chunk
        const float Et = fact ? sm.E[t] : 1.0f;
        // D x enters as D / E_t on the diagonal of M (x_t is an exact operand of that product)
        const float Ddiag = Dh / Et;
        f32x4v yd = {0.0f, 0.0f, 0.0f, 0.0f};
        bf16x8 cn[N / 32];  // C rows 16 tt .., natural k = n order
#pragma unroll
        for (int k = 0; k < N / 32; ++k) cn[k] = operand(sm.cs, PN, 16 * tt, 32 * k);
        const float cum_t = fact ? 0.0f : sm.cum[t];
#pragma unroll
        for (int kk = 0; kk <= tt / 2; ++kk) {
            float m[8];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int st = 2 * kk + half;
                if (st > tt) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) m[4 * half + j] = 0.0f;
                    continue;
                }
                f32x4v gt = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int k = 0; k < N / 32; ++k) gt = mfma(operand(sm.bs, PN, 16 * st, 32 * k), cn[k], gt);
                const int s0 = 16 * st + 4 * (l >> 4);  // this lane's rows s0 .. s0 + 3
                if (fact) {
                    const f32x4v F = *reinterpret_cast<const f32x4v*>(sm.F + s0);
#pragma unroll
                    for (int j = 0; j < 4; ++j) m[4 * half + j] = gt[j] * F[j];
                } else {
                    const f32x4v cs4 = *reinterpret_cast<const f32x4v*>(sm.cum + s0);
                    const f32x4v dl4 = *reinterpret_cast<const f32x4v*>(sm.dl + s0);
#pragma unroll
                    for (int j = 0; j < 4; ++j) m[4 * half + j] = gt[j] * (fast_exp2(A2 * (cum_t - cs4[j])) * dl4[j]);
                }
                if (st == tt) {  // the diagonal tile: s <= t only, and D / E_t at s = t
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        m[4 * half + j] = s0 + j < t ? m[4 * half + j] : (s0 + j == t ? m[4 * half + j] + Ddiag : 0.0f);
                }
            }
            bf16x8 mh, ml;
            split8(m[0], m[1], m[2], m[3], m[4], m[5], m[6], m[7], mh, ml);
            const bf16x8& xo = kk == 0 ? xo0 : xo1;
            yd = mfma(xo, mh, yd);
            yd = mfma(xo, ml, yd);
        }
        // out: channels 16 w + 4 (l / 16) + j at time step t
        const float Eo = sm.Eo[t];
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v = fmaf(Et, yd[j], Eo * yo[tt][j]);
            if (HAS_Z) {
                const uint32_t zw = zc[tt][j >> 1];
                v *= silu((j & 1) ? bf_hi(zw) : bf_lo(zw));
            }
            o[j] = v;
        }
        if (FAST || t < valid)
            *reinterpret_cast<u32x2*>(orow + static_cast<int64_t>(16 * tt) * H * kP) =
                u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
    }
}

template <int N, bool HAS_Z>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(N == 64 ? 3 : 2))) void ssd_main_kernel(SsdArgs a) {
    __shared__ __align__(16) Smem<N, true> sm;
    const int seg = blockIdx.x, h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int g = h / (a.H / a.G);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const float A2 = a.A[h] * kLog2e;
    const float Dh = a.D ? a.D[h] : 0.0f;
    const float bias = a.bias ? a.bias[h] : 0.0f;
    const int64_t c0 = seg * a.nchunks / a.S, c1 = (seg + 1) * a.nchunks / a.S;
    const int64_t bh_row = b * a.L * a.H + h, bg_row = b * a.L * a.G + g;

    // the state entering the segment: the earlier segments' local end states folded in order
    f32x4v hacc[N / 16];
#pragma unroll
    for (int i = 0; i < N / 16; ++i) hacc[i] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = 0; k < seg; ++k) {
        const float* src = seg_slot(a, b, h, k, N);
        const float e = fast_exp2(A2 * src[kP * N]);
        src += w * (N / 16) * 4 * 64 + l;
#pragma unroll
        for (int i = 0; i < N / 16; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) hacc[i][j] = fmaf(e, hacc[i][j], src[(4 * i + j) * 64]);
    }

    Tiles<N> nxt;
    if (c0 < c1) load_tiles<N, true>(nxt, a, bh_row, bg_row, c0);
    for (int64_t c = c0; c < c1; ++c) {
        __syncthreads();  // the previous chunk's reads of the staged tiles are done
        u32x2 zc[4];      // z of this chunk, consumed by the epilogues
        if (HAS_Z) load_rows4(zc, a.z, a, bh_row, c * kQ);
        const ChunkInfo ci = stage_tiles<N, true>(sm, nxt, a, A2, bias, c);
        __syncthreads();
        // The next chunk's tiles (the last chunk reloads its own, from the cache): a load on every
        // path keeps the compiler's count of outstanding loads exact, so waiting for z below does
        // not also wait for these.
        load_tiles<N, true>(nxt, a, bh_row, bg_row, c + 1 < c1 ? c + 1 : c);

        // this lane's output row of the chunk for t-tile 0: time step l % 16, channels 16 w + 4 (l / 16) ..
        uint16_t* const orow = a.out + (bh_row + (c * kQ + (l & 15)) * a.H) * kP + 16 * w + 4 * (l >> 4);
        if (ci.fact && (c + 1) * kQ <= a.L)
            chunk_outputs<N, HAS_Z, true>(sm, ci, hacc, zc, A2, Dh, orow, a.H, kQ);
        else
            chunk_outputs<N, HAS_Z, false>(sm, ci, hacc, zc, A2, Dh, orow, a.H, a.L - c * kQ);
        // the state for the next chunk (the staged tiles stay until the next chunk's first barrier)
        state_step<N, true>(sm, hacc, ci.eend);
    }
    if (a.last_state && seg == a.S - 1) {
        // H^T[n][p] of this wavefront: n = 16 i + 4 (l / 16) + j, p = 16 w + l % 16
        float* dst = a.last_state + (b * a.H + h) * kP * N + (16 * w + (l & 15)) * N + 4 * (l >> 4);
#pragma unroll
        for (int i = 0; i < N / 16; ++i)
            *reinterpret_cast<f32x4v*>(dst + 16 * i) = hacc[i];
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

// Segments per (batch, head): about four workgroups per CU in all, at least two chunks each.
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
