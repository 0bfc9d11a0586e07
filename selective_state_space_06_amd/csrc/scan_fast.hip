// scan_fast.hip -- forward selective scan (S6), the fast path for 16-byte-aligned rows.
//
// Same computation as scan_fwd.hip (Mamba paper Section 3 / Algorithm 2 as coded on the
// Keras/TensorFlow Mamba tutorial page: delta = softplus(delta_raw + bias), Abar = exp(delta A),
// h_t = Abar h_{t-1} + delta B u, out = (C.h + D u) silu(z)), organised for gfx950:
//
//   * lane = channel: each of the 64 lanes of a wavefront owns one (b, d) row and keeps its 16
//     states in VGPRs; the wave walks its time segment sequentially, two steps per iteration of
//     a loop that is deliberately not unrolled further (so the compiler cannot interleave the
//     independent per-step work of many steps and run out of registers);
//   * u / delta stream in as 16-byte vectors of the lane's own row, a 64-byte tile (32 bf16 or
//     16 fp32 steps) at a time; the next tile is prefetched into VGPRs while the current one
//     runs from LDS, stored word-major ([word][lane]) so every per-step LDS access of the wave
//     hits 64 distinct banks;
//   * B_t and C_t are shared by the 64 lanes of a wave (one batch).  Per tile, the wave loads
//     the (N, tile) blocks of B and C straight from their (Bt, N, L) layout (prefetched with the
//     u / delta tile) and stores them time-major in LDS; each step reads its B_t | C_t as eight
//     16-byte broadcast loads (all lanes one address) into plain VGPR operands.  (Feeding them
//     through DPP row broadcasts instead saves those loads but stops the SIMD from dual-issuing
//     VALU work of different waves, which costs more than it saves.)
//   * the per-step result y + D u stays fp32 in the LDS words the step has consumed; an
//     epilogue per tile applies the gate silu(z) (z of the tile is loaded into VGPRs when the
//     tile starts), rounds to the storage type and writes 16-byte vectors;
//   * the work is spread over one round of wavefronts for the whole chip: the (64-channel group,
//     tile) pairs of the call are numbered group-major and each wavefront takes an equal
//     contiguous range of them, so no SIMD holds more work than another.  A range that starts
//     inside a group needs the state reached there: a first kernel computes, for every range
//     that ends inside a group, the pair (sum of delta, end state from h = 0) of that last piece;
//     the main kernel folds the pairs of the group's earlier pieces with the associative operator
//     (a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2) into its starting state and runs its piece.
//     A scan continued from a given state h0 starts that fold from h0 instead of zeros (the
//     aggregates do not depend on it).  With per-batch sequence lengths, the steps at or past a
//     batch's length get dt = 0 (abar = 1, no input: the state stands still) and zero outputs, so
//     the aggregates, the fold and the final state need no other change.
//
// exp is exp2 of a log2(e)-prescaled argument.  When every row of a wave satisfies
// A[d, n] == (n + 1) A[d, 0] exactly (the S4D-real A = -(1..N) of the tutorial's init),
// Abar_n = Abar_0^(n+1) is formed by multiplications (one exp2 per (b, d, t)); the aggregate
// pass then uses the backward form sum_s x_s B_s R_s^(n+1), R_s the product of the later
// Abar_0, which costs two VALU operations per state update.
#include "device_math.hpp"
#include "mss_internal.hpp"

namespace mss {
namespace {

template <class E>
struct Geo {
    static constexpr int V = E::kPerVec;             // elements per 16 bytes
    static constexpr int BYTES = fast_tile_bytes(V == 8);
    static constexpr int NV = BYTES / 16;            // 16-byte vectors per row and array in a tile
    static constexpr int TT = NV * V;                // steps per tile
    static constexpr int W = BYTES / 4;              // words per row and array
    static constexpr int kBCChunks = TT / 8;       // 16-byte B|C chunks per lane
    static constexpr int kRowWords = 2 * W * 64;   // u and delta, [word][lane]
};

struct RowSetup {
    int64_t row;      // flat (b, d) row, clamped to a valid row for inactive lanes
    bool active;      // lane maps to a real channel
    float A2[kN];     // A[d, n] * log2(e)
    float bias, dskip;
    bool pow_ok;
    int64_t stop;     // the batch's sequence length (steps at or past it are identity steps)
};

__device__ __forceinline__ RowSetup row_setup(const float* __restrict__ A, const float* __restrict__ D,
                                              const float* __restrict__ bias, int64_t Dn,
                                              const int32_t* __restrict__ lens, int64_t L, int64_t cb,
                                              int64_t b) {
    RowSetup r;
    if (lens) {
        const int64_t l = lens[b];
        r.stop = l < 0 ? 0 : (l > L ? L : l);
    } else {
        r.stop = L;
    }
    const int64_t d = cb * 64 + threadIdx.x;
    r.active = d < Dn;
    const int64_t dc = r.active ? d : Dn - 1;
    r.row = b * Dn + dc;
    const float4* Ar = reinterpret_cast<const float4*>(A + dc * kN);
    float Av[kN];
#pragma unroll
    for (int q = 0; q < kN / 4; ++q) {
        const float4 v = Ar[q];
        Av[4 * q] = v.x; Av[4 * q + 1] = v.y; Av[4 * q + 2] = v.z; Av[4 * q + 3] = v.w;
    }
    r.pow_ok = true;
#pragma unroll
    for (int n = 0; n < kN; ++n) {
        r.A2[n] = Av[n] * kLog2e;
        r.pow_ok = r.pow_ok && (Av[n] == static_cast<float>(n + 1) * Av[0]);
    }
    r.bias = bias ? bias[dc] : 0.0f;
    r.dskip = D ? D[dc] : 0.0f;
    return r;
}

// One tile of this lane's row of u and delta as loaded from HBM (plain words: an array of vector
// structs here ends up in scratch memory).
template <class E>
struct RawUD {
    uint32_t u[4 * Geo<E>::NV], d[4 * Geo<E>::NV];
};

// The 16-byte vector of row rp at step t.  RAGGED (rows of any length, so only element-aligned):
// an unaligned 16-byte load (gfx950 serves it whole), and a vector running past the row's end
// L is read element by element with zeros after the end, so no load leaves the row's tensor.
// (t and L are the same for every lane: the choice is uniform.)
template <class E, bool RAGGED>
__device__ __forceinline__ uint4 load_vec(const typename E::storage* __restrict__ rp, int64_t t, int64_t L) {
    constexpr int V = E::kPerVec;
    if (!RAGGED) return *reinterpret_cast<const uint4*>(rp + t);
    if (t + V <= L) {
        uint4 w;
        __builtin_memcpy(&w, rp + t, 16);
        return w;
    }
    float f[V];
#pragma unroll
    for (int e = 0; e < V; ++e) f[e] = t + e < L ? E::load1(rp, t + e) : 0.0f;
    return E::pack(f);  // exact: the values came from this storage type
}

// An element-aligned 16-byte access (RAGGED rows; gfx950 serves it whole).
__device__ __forceinline__ uint4 load16u(const void* p) {
    uint4 w;
    __builtin_memcpy(&w, p, 16);
    return w;
}

// Vectors at or past t_end re-read the last valid vector (their steps are never used), so every
// load is unconditional and in bounds.  RAGGED: vectors past the row's end read as zeros; a tile
// that lies wholly inside the row (all but a row's last) takes plain element-aligned loads with
// no per-vector test, so they issue together (the tested form waits on each load in turn).
template <class E, bool RAGGED>
__device__ __forceinline__ void load_ud(RawUD<E>& r, const typename E::storage* __restrict__ up,
                                        const typename E::storage* __restrict__ dp, int64_t t0,
                                        int64_t t_end, int64_t L) {
    constexpr int V = E::kPerVec;
    if (RAGGED && t0 + Geo<E>::TT <= L) {
#pragma unroll
        for (int v = 0; v < Geo<E>::NV; ++v) {
            const uint4 a = load16u(up + t0 + v * V);
            const uint4 b = load16u(dp + t0 + v * V);
            r.u[4 * v] = a.x; r.u[4 * v + 1] = a.y; r.u[4 * v + 2] = a.z; r.u[4 * v + 3] = a.w;
            r.d[4 * v] = b.x; r.d[4 * v + 1] = b.y; r.d[4 * v + 2] = b.z; r.d[4 * v + 3] = b.w;
        }
        return;
    }
#pragma unroll
    for (int v = 0; v < Geo<E>::NV; ++v) {
        int64_t t = t0 + v * V;
        if (!RAGGED) t = t < t_end ? t : t_end - V;
        const uint4 a = load_vec<E, RAGGED>(up, t, L);
        const uint4 b = load_vec<E, RAGGED>(dp, t, L);
        r.u[4 * v] = a.x; r.u[4 * v + 1] = a.y; r.u[4 * v + 2] = a.z; r.u[4 * v + 3] = a.w;
        r.d[4 * v] = b.x; r.d[4 * v + 1] = b.y; r.d[4 * v + 2] = b.z; r.d[4 * v + 3] = b.w;
    }
}

// Word-major staging: word w of lane l at srow[w * 64 + l]; delta follows u after W words.
template <class E>
__device__ __forceinline__ void stage_ud(uint32_t* srow, const RawUD<E>& r) {
    constexpr int W = Geo<E>::W;
#pragma unroll
    for (int w = 0; w < W; ++w) {
        srow[w * 64 + threadIdx.x] = r.u[w];
        srow[(W + w) * 64 + threadIdx.x] = r.d[w];
    }
}

// The tile's B and C blocks: chunk k of lane l is the 16-byte run of B (k < K/2) or C at
// n = l % 16, steps t0 + 4 * (4 (k % (K/2)) + l / 16) .. + 3.  Runs at or past t_end are clamped
// to the last four valid steps (t_end is a multiple of 4 here).
template <class E>
struct RawBC {
    uint32_t w[4 * Geo<E>::kBCChunks];
};

template <class E, bool WITH_C, bool RAGGED>
__device__ __forceinline__ void load_bc(RawBC<E>& r, const float* __restrict__ Bb,
                                        const float* __restrict__ Cb, int64_t L, int64_t t0,
                                        int64_t t_end) {
    constexpr int K = Geo<E>::kBCChunks;
    const int n = threadIdx.x & 15;
    const bool whole = RAGGED && t0 + Geo<E>::TT <= L;  // the tile lies inside the rows (uniform)
#pragma unroll
    for (int k = 0; k < (WITH_C ? K : K / 2); ++k) {
        const float* src = k < K / 2 ? Bb : Cb;
        const int kk = k % (K / 2);
        int64_t t = t0 + 4 * (4 * kk + (threadIdx.x >> 4));
        if (!RAGGED) t = t < t_end ? t : t_end - 4;
        const uint4 v = whole ? load16u(src + n * L + t) : load_vec<F32, RAGGED>(src + n * L, t, L);
        r.w[4 * k] = v.x; r.w[4 * k + 1] = v.y; r.w[4 * k + 2] = v.z; r.w[4 * k + 3] = v.w;
    }
}

// Time-major LDS block: step t of the tile at sbc + t * SB, B_t in floats [0, 16), C_t in
// [16, 32).  SB = 16 (B only) + 4 or 32 + 4: the 4 spare floats per step put the 16 lanes x 4
// step groups of each scattered 4-byte store in 64 distinct banks.
// VARLEN: B and C at or past the batch's length stage as zeros, so whatever the tensors hold
// there (padding) cannot reach the state through x B with x = 0.
template <class E, bool WITH_C, bool VARLEN>
__device__ __forceinline__ void stage_bc(float* sbc, const RawBC<E>& r, int64_t t0, int64_t stop) {
    constexpr int K = Geo<E>::kBCChunks;
    constexpr int SB = WITH_C ? 36 : 20;
    const int n = threadIdx.x & 15;
#pragma unroll
    for (int k = 0; k < (WITH_C ? K : K / 2); ++k) {
        const int kk = k % (K / 2);
        const int t = 4 * (4 * kk + (threadIdx.x >> 4));
        float* dst = sbc + t * SB + (k < K / 2 ? 0 : kN) + n;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = __uint_as_float(r.w[4 * k + i]);
            dst[i * SB] = (VARLEN && t0 + t + i >= stop) ? 0.0f : v;
        }
    }
}

template <bool SOFTPLUS>
__device__ __forceinline__ float delta_of(float raw, float bias) {
    const float pre = raw + bias;
    return SOFTPLUS ? softplus(pre) : pre;
}

// Elements j, j + 1 (j even) of the lane's staged row of one array.
template <class E>
__device__ __forceinline__ void staged2(const uint32_t* arr, int j, float& e0, float& e1) {
    if (E::kPerVec == 8) {
        const uint32_t w = arr[(j >> 1) * 64 + threadIdx.x];
        e0 = bf16_lo(w);
        e1 = bf16_hi(w);
    } else {
        e0 = __uint_as_float(arr[j * 64 + threadIdx.x]);
        e1 = __uint_as_float(arr[(j + 1) * 64 + threadIdx.x]);
    }
}

// Per-step scalars of the step pair (j, j + 1): delta, x = delta u, Abar_0 = exp2(delta A2_0)
// (power path) and D u (main kernel).  The loops compute the pair after next while the current
// pair's state updates run, so the softplus / exp2 latency of one pair overlaps the other's work.
struct Pair {
    float d[2], x[2], a[2], du[2];
};

// The main kernel's power path keeps the state scaled: the lane holds g = h / sc, sc the scale
// of the step last taken (1 where the state was set).  Step t takes the scale s_t = step_scale(x_t)
// = x_t + copysign(2^-40, x_t), never zero, and computes g_t = (sc / s_t) a^(n+1) g_(t-1) + B_t
// and y_t = s_t (C_t . g_t) + D u_t: B enters the state update without a multiplication by x (16
// fewer per step).  This adds s_t B_t instead of x_t B_t, 2^-40 |B_t| per state and step away
// from the recurrence: an absolute deviation far below what the fp32 state resolves at the
// magnitudes the tolerances allow (identity steps past a sequence's end stage B as 0 and add
// nothing).  |g| <= |h| 2^40 keeps g far from overflow.  Every kernel variant forms the same s
// from the same x, so a scan with per-batch lengths equal to L gives the plain scan's results
// bit for bit.

template <class E, bool SOFTPLUS, bool POW, bool WITH_DU, bool VARLEN = false>
__device__ __forceinline__ Pair pair_of(const uint32_t* su, const uint32_t* sd, int j, const RowSetup& rs,
                                        int64_t t0 = 0) {
    Pair p;
    float u[2], r[2];
    staged2<E>(su, j, u[0], u[1]);
    staged2<E>(sd, j, r[0], r[1]);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        p.d[i] = delta_of<SOFTPLUS>(r[i], rs.bias);
        p.x[i] = p.d[i] * u[i];
        if (VARLEN && t0 + j + i >= rs.stop) p.d[i] = p.x[i] = 0.0f;  // past the sequence: an identity step
        p.a[i] = POW ? fast_exp2(p.d[i] * rs.A2[0]) : 0.0f;
        p.du[i] = WITH_DU ? rs.dskip * u[i] : 0.0f;
    }
    return p;
}

// Step results j, j + 1 (fp32) written into words the step pair has consumed: bf16 puts them in
// the u and delta words j / 2, fp32 in the u words j and j + 1.
template <class E>
__device__ __forceinline__ void put2(uint32_t* srow, int j, float o0, float o1) {
    constexpr int W = Geo<E>::W;
    if (E::kPerVec == 8) {
        srow[(j >> 1) * 64 + threadIdx.x] = __float_as_uint(o0);
        srow[(W + (j >> 1)) * 64 + threadIdx.x] = __float_as_uint(o1);
    } else {
        srow[j * 64 + threadIdx.x] = __float_as_uint(o0);
        srow[(j + 1) * 64 + threadIdx.x] = __float_as_uint(o1);
    }
}

// Step result e of the tile as written by put2.
template <class E>
__device__ __forceinline__ float result_of(const uint32_t* srow, int e) {
    constexpr int W = Geo<E>::W;
    if (E::kPerVec == 8)
        return __uint_as_float(srow[((e & 1) ? W + (e >> 1) : (e >> 1)) * 64 + threadIdx.x]);
    return __uint_as_float(srow[e * 64 + threadIdx.x]);
}

// Element e of the 16-byte vector held in words w[0..3].
template <class E>
__device__ __forceinline__ float vec_elem(const uint32_t* w, int e) {
    if (E::kPerVec == 8) return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
    return __uint_as_float(w[e]);
}

// Powers a^1 .. a^16 with a multiplication tree of depth 4 (15 multiplications).
__device__ __forceinline__ void powers16(float a, float (&p)[kN]) {
    p[0] = a;
    p[1] = a * a;
    p[2] = p[1] * a;
    p[3] = p[1] * p[1];
#pragma unroll
    for (int k = 0; k < 4; ++k) p[4 + k] = p[3] * p[k];
#pragma unroll
    for (int k = 0; k < 8; ++k) p[8 + k] = p[7] * p[k];
}

// One time step for one lane: 16 state updates and y0 + C.h; bc = B_t | C_t in LDS; a = Abar_0
// on the power path.
template <bool POW>
__device__ __forceinline__ float step_main(float (&h)[kN], const float (&A2)[kN], float dl, float x,
                                           float a, const float* bc, float y0) {
    const float4* b4 = reinterpret_cast<const float4*>(bc);
    float bv[kN], cv[kN];
#pragma unroll
    for (int q = 0; q < kN / 4; ++q) {
        const float4 b = b4[q], c = b4[kN / 4 + q];
        bv[4 * q] = b.x; bv[4 * q + 1] = b.y; bv[4 * q + 2] = b.z; bv[4 * q + 3] = b.w;
        cv[4 * q] = c.x; cv[4 * q + 1] = c.y; cv[4 * q + 2] = c.z; cv[4 * q + 3] = c.w;
    }
    float y1 = 0.0f;
    if (POW) {
        float p[kN];
        powers16(a, p);
#pragma unroll
        for (int n = 0; n < kN; ++n) {
            h[n] = fmaf(p[n], h[n], x * bv[n]);
            if (n & 1) y1 = fmaf(cv[n], h[n], y1);
            else y0 = fmaf(cv[n], h[n], y0);
        }
    } else {
#pragma unroll
        for (int n = 0; n < kN; ++n) {
            h[n] = fmaf(fast_exp2(dl * A2[n]), h[n], x * bv[n]);
            if (n & 1) y1 = fmaf(cv[n], h[n], y1);
            else y0 = fmaf(cv[n], h[n], y0);
        }
    }
    return y0 + y1;
}

// One scaled step (power path): g = r a^(n+1) g + B_t with r = sc / s_t, returns
// s_t (C_t . g) + D u_t.  The factors r a^(n+1) come from r a by doubling (a^2, a^4, a^8): 19
// multiplications where the plain step takes 15 for the powers and 16 for x B.
__device__ __forceinline__ float step_scaled(float (&g)[kN], float r, float a, float st, const float* bc,
                                             float du) {
    const float4* b4 = reinterpret_cast<const float4*>(bc);
    float bv[kN], cv[kN];
#pragma unroll
    for (int q = 0; q < kN / 4; ++q) {
        const float4 b = b4[q], c = b4[kN / 4 + q];
        bv[4 * q] = b.x; bv[4 * q + 1] = b.y; bv[4 * q + 2] = b.z; bv[4 * q + 3] = b.w;
        cv[4 * q] = c.x; cv[4 * q + 1] = c.y; cv[4 * q + 2] = c.z; cv[4 * q + 3] = c.w;
    }
    float f[kN];
    const float a2 = a * a, a4 = a2 * a2, a8 = a4 * a4;
    f[0] = r * a;
    f[1] = f[0] * a;
    f[2] = f[0] * a2;
    f[3] = f[1] * a2;
#pragma unroll
    for (int k = 0; k < 4; ++k) f[4 + k] = f[k] * a4;
#pragma unroll
    for (int k = 0; k < 8; ++k) f[8 + k] = f[k] * a8;
    float y0 = 0.0f, y1 = 0.0f;
#pragma unroll
    for (int n = 0; n < kN; ++n) {
        g[n] = fmaf(f[n], g[n], bv[n]);
        if (n & 1) y1 = fmaf(cv[n], g[n], y1);
        else y0 = fmaf(cv[n], g[n], y0);
    }
    return fmaf(st, y0 + y1, du);
}

// Steps the loops of a tile run: a multiple of 4 (RAGGED: rounded up; the extra steps lie past
// the row's end and are identity steps).
template <bool RAGGED, int TT>
__device__ __forceinline__ int tile_steps(int64_t t0, int64_t t_end) {
    const int64_t n = t_end - t0 < TT ? t_end - t0 : TT;
    return static_cast<int>(RAGGED ? ((n + 3) & ~static_cast<int64_t>(3)) : n);
}

template <class E, bool HAS_Z, bool SOFTPLUS, bool POW, bool VARLEN, bool RAGGED, bool SAVE>
__device__ __forceinline__ void main_body(
    const RowSetup& rs, float (&h)[kN], const typename E::storage* __restrict__ up,
    const typename E::storage* __restrict__ dp, const typename E::storage* __restrict__ zp,
    typename E::storage* __restrict__ op, const float* __restrict__ Bb, const float* __restrict__ Cb,
    int64_t L, uint32_t* srow, float* sbc, int64_t t_begin, int64_t t_end, float* saved, int64_t R) {
    using G = Geo<E>;
    constexpr int V = G::V, TT = G::TT, W = G::W;
    const uint32_t* su = srow;
    const uint32_t* sd = srow + W * 64;
    float* const srow_saved = SAVE ? saved + rs.row * 4 : nullptr;  // this lane's float4 in each plane
    constexpr int kNV = G::NV;
    RawUD<E> pre;
    RawBC<E> bpre;
    // bf16 rows on the power path take the scaled steps (h = sc * g, the array h holding g).
    // fp32 rows run one wavefront per SIMD and wait on memory more than they issue: there the
    // reciprocal's latency in the chain cost more than the 16 multiplications it saves.
    constexpr bool SCALED = POW && V == 8;
    float sc = 1.0f;
    load_ud<E, RAGGED>(pre, up, dp, t_begin, t_end, L);
    load_bc<E, true, RAGGED>(bpre, Bb, Cb, L, t_begin, t_end);
    for (int64_t t0 = t_begin; t0 < t_end; t0 += TT) {
        __syncthreads();  // the previous tile's reads of the shared B|C block are done
        stage_ud<E>(srow, pre);
        stage_bc<E, true, VARLEN>(sbc, bpre, t0, rs.stop);
        __syncthreads();
        uint32_t zw[4 * kNV];  // z of this tile, consumed by the epilogue
        const bool whole = RAGGED && t0 + TT <= L;  // the tile lies inside the row (uniform)
        if (HAS_Z) {
#pragma unroll
            for (int v = 0; v < kNV; ++v) {
                int64_t t = t0 + v * V;
                if (!RAGGED) t = t < t_end ? t : t_end - V;
                const uint4 a = whole ? load16u(zp + t) : load_vec<E, RAGGED>(zp, t, L);
                zw[4 * v] = a.x; zw[4 * v + 1] = a.y; zw[4 * v + 2] = a.z; zw[4 * v + 3] = a.w;
            }
        }
        if (t0 + TT < t_end) {
            load_ud<E, RAGGED>(pre, up, dp, t0 + TT, t_end, L);
            load_bc<E, true, RAGGED>(bpre, Bb, Cb, L, t0 + TT, t_end);
        }
        const int nsteps = tile_steps<RAGGED, TT>(t0, t_end);  // multiple of 4
        Pair cur = pair_of<E, SOFTPLUS, POW, true, VARLEN>(su, sd, 0, rs, t0);
        // Two step pairs per iteration on the scaled path (no copies of the next pair's scalars: the
        // two register sets alternate; 138.9 against 142.1 us on the 2.8B layer); one elsewhere
        // (the random-A path unrolled is slower: 176.0 against 173.5 us).
        constexpr int kUnroll = SCALED ? 2 : 1;
#pragma unroll kUnroll
        for (int j = 0; j < nsteps; j += 2) {
            // for the backward: the state entering each 8-step tile (tiles start on multiples of 8)
            if (SAVE && (j & 7) == 0 && t0 + j < L && rs.active) {
                // planes of float4 (states 4q..4q+3 of every row): a wave writes 1 KiB runs,
                // streamed past the caches (read back only by the backward)
                f32x4* sp = reinterpret_cast<f32x4*>(srow_saved + ((t0 + j) >> 3) * kN * R);
#pragma unroll
                for (int q = 0; q < kN / 4; ++q) {  // h = sc g (sc stays 1 off the scaled path)
                    const f32x4 v = {sc * h[4 * q], sc * h[4 * q + 1], sc * h[4 * q + 2], sc * h[4 * q + 3]};
                    __builtin_nontemporal_store(v, sp + q * R);
                }
            }
            // the last iteration recomputes its own pair (read before put2 overwrites it)
            const Pair nxt =
                pair_of<E, SOFTPLUS, POW, true, VARLEN>(su, sd, j + 2 < nsteps ? j + 2 : j, rs, t0);
            float y0, y1;
            if (SCALED) {
                const float s0 = step_scale(cur.x[0]);
                const float s1 = step_scale(cur.x[1]);
                y0 = step_scaled(h, sc * fast_rcp(s0), cur.a[0], s0, sbc + j * 36, cur.du[0]);
                y1 = step_scaled(h, s0 * fast_rcp(s1), cur.a[1], s1, sbc + (j + 1) * 36, cur.du[1]);
                sc = s1;
            } else {
                y0 = step_main<POW>(h, rs.A2, cur.d[0], cur.x[0], cur.a[0], sbc + j * 36, cur.du[0]);
                y1 = step_main<POW>(h, rs.A2, cur.d[1], cur.x[1], cur.a[1], sbc + (j + 1) * 36, cur.du[1]);
            }
            put2<E>(srow, j, y0, y1);
            cur = nxt;
        }
        // Epilogue: gate and round the whole tile first (one block of independent work the
        // compiler can interleave), then the 16-byte stores of the valid vectors.
        uint4 packed[kNV];
#pragma unroll
        for (int v = 0; v < kNV; ++v) {
            float o[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                o[e] = result_of<E>(srow, v * V + e);
                if (HAS_Z) o[e] *= silu(vec_elem<E>(zw + 4 * v, e));
                if (VARLEN && t0 + v * V + e >= rs.stop) o[e] = 0.0f;
            }
            packed[v] = E::pack(o);
        }
        if (rs.active && RAGGED && t0 + TT <= t_end) {  // every vector of the tile is the row's
#pragma unroll
            for (int v = 0; v < kNV; ++v) __builtin_memcpy(op + t0 + v * V, &packed[v], 16);
        } else if (rs.active) {
#pragma unroll
            for (int v = 0; v < kNV; ++v) {
                const int64_t t = t0 + v * V;
                if (!RAGGED) {
                    if (t < t_end) *reinterpret_cast<uint4*>(op + t) = packed[v];
                } else if (t + V <= t_end) {
                    __builtin_memcpy(op + t, &packed[v], 16);  // element-aligned 16-byte store
                } else if (t < t_end) {  // the row's last, partial vector: only its own elements
#pragma unroll
                    for (int e = 0; e < V; ++e)
                        if (t + e < t_end) E::store1(op, t + e, vec_elem<E>(&packed[v].x, e));
                }
            }
        }
    }
    if (SCALED) {
#pragma unroll
        for (int n = 0; n < kN; ++n) h[n] *= sc;  // back to the state itself
    }
}

// The work of a call is the grid of (channel group, tile) pairs: G groups of 64 rows (a group is
// one batch's channel block cb, g = b * gx + cb) times T = ceil(L / TT) tiles each, numbered
// group-major.  With GT = q W + rem, wavefront w of W takes the contiguous range starting at
// w q + min(w, rem), q + 1 tiles for the first rem wavefronts and q for the others, so every
// wavefront gets the same number of tiles to within one.  A range can start
// in the middle of a group (its first piece then needs the state reached at that tile) and can
// run on into the next group (whose first tile starts from h0 / zeros).  W is one full round of
// wavefronts for the chip, so no SIMD ends up with more wavefronts than another.
//
// Wavefront numbers are dealt to the XCDs in contiguous blocks.  The hardware hands consecutive
// workgroups to the XCDs in turn (workgroup i to XCD i mod X), so workgroup i takes number
// xcd * q + min(xcd, r) + i / X, with W = q X + r: XCD k then scans one contiguous stretch of
// groups, and its L2 and address translation see 1/X of the rows instead of all of them
// (measured: 12-24% faster than numbering the wavefronts in workgroup order).
// Every count below the tile count is held in 32 bits (the host refuses a plan whose counts do
// not fit), so the divisions of the per-piece set-up stay short.
struct Part {
    uint32_t T;    // tiles per group
    uint32_t W;    // wavefronts, 1 <= W <= G T
    uint32_t q;    // G T / W
    uint32_t rem;  // G T mod W
    uint32_t gx;   // channel groups per batch
    uint32_t xq, xr;  // W = xq X + xr: wavefronts per XCD (the first xr XCDs take one more)
    uint32_t X;    // XCDs the workgroups are dealt over
};

__device__ __forceinline__ uint32_t part_begin(const Part& p, uint32_t w) {
    return w * p.q + (w < p.rem ? w : p.rem);
}

// This workgroup's wavefront number (a bijection of [0, W)).
__device__ __forceinline__ uint32_t wave_of(const Part& p) {
    const uint32_t i = blockIdx.x, x = i % p.X;
    return x * p.xq + (x < p.xr ? x : p.xr) + i / p.X;
}

// The wavefront whose range holds tile t of the numbering.  For t = g T, the start of group g,
// its range and those of the wavefronts up to the one holding tile r cover group g's tiles
// before r.
__device__ __forceinline__ uint32_t wave_holding(const Part& p, uint32_t t) {
    const uint32_t big = p.rem * (p.q + 1);  // tiles of the wavefronts that take q + 1
    return t < big ? t / (p.q + 1) : p.rem + (t - big) / p.q;
}

// Where wavefront w's aggregate lives: one slot per wavefront, [slot][n (16 states, then the sum of
// delta)][lane], so a wave's loads of one word are 256 contiguous bytes.
__device__ __forceinline__ const float* agg_slot(const float* agg, uint32_t w) {
    return agg + static_cast<size_t>(w) * (kN + 1) * 64 + threadIdx.x;
}

// B at steps j, j + 1 from the aggregate kernel's B block (stride 20 floats per step).
struct BPair {
    float b[2][kN];
};

__device__ __forceinline__ BPair b_pair(const float* sbc, int j) {
    BPair r;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float4* p = reinterpret_cast<const float4*>(sbc + (j + i) * 20);
#pragma unroll
        for (int q = 0; q < kN / 4; ++q) {
            const float4 v = p[q];
            r.b[i][4 * q] = v.x; r.b[i][4 * q + 1] = v.y; r.b[i][4 * q + 2] = v.z; r.b[i][4 * q + 3] = v.w;
        }
    }
    return r;
}

// Folds the aggregates of slots [s_begin, s_end) (the pieces of this group before the current
// one, in order) into the starting state, four slots per round: the 68 loads of a round are
// issued together, so a round costs one memory round trip.  The fold starts from the row's h0
// when one is given, else from zeros.
template <bool POW>
__device__ __forceinline__ void fold_carry(float (&h)[kN], const float (&A2)[kN],
                                           const float* __restrict__ agg, const float* __restrict__ h0,
                                           uint32_t s_begin, uint32_t s_end, int64_t row) {
    constexpr int kRound = 4;
    if (h0) {
        const float4* src = reinterpret_cast<const float4*>(h0 + row * kN);
#pragma unroll
        for (int q = 0; q < kN / 4; ++q) {
            const float4 v = src[q];
            h[4 * q] = v.x; h[4 * q + 1] = v.y; h[4 * q + 2] = v.z; h[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int n = 0; n < kN; ++n) h[n] = 0.0f;
    }
    for (uint32_t s0 = s_begin; s0 < s_end; s0 += kRound) {
        float v[kRound][kN + 1];
#pragma unroll
        for (int i = 0; i < kRound; ++i) {
            const uint32_t s = s0 + i < s_end ? s0 + i : s_end - 1;  // past the end: reload the last one
            const float* a = agg_slot(agg, s);
#pragma unroll
            for (int n = 0; n <= kN; ++n) v[i][n] = a[n * 64];
        }
#pragma unroll
        for (int i = 0; i < kRound; ++i) {
            if (s0 + i < s_end) {
                if (POW) {
                    float p[kN];
                    powers16(fast_exp2(v[i][kN] * A2[0]), p);
#pragma unroll
                    for (int n = 0; n < kN; ++n) h[n] = fmaf(p[n], h[n], v[i][n]);
                } else {
#pragma unroll
                    for (int n = 0; n < kN; ++n) h[n] = fmaf(fast_exp2(v[i][kN] * A2[n]), h[n], v[i][n]);
                }
            }
        }
    }
}

template <class E, bool HAS_Z, bool SOFTPLUS, bool VARLEN, bool RAGGED, bool SAVE>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void scan_main_kernel(
    const typename E::storage* __restrict__ u, const typename E::storage* __restrict__ delta,
    const typename E::storage* __restrict__ z, const float* __restrict__ A,
    const float* __restrict__ B, const float* __restrict__ C, const float* __restrict__ D,
    const float* __restrict__ bias, const float* __restrict__ agg, const float* __restrict__ h0,
    typename E::storage* __restrict__ out, float* __restrict__ last_state, const int32_t* __restrict__ lens,
    float* __restrict__ saved, int64_t Dn, int64_t L, int64_t R, Part p) {
    using G = Geo<E>;
    __shared__ uint32_t srow[G::kRowWords];
    __shared__ __align__(16) float sbc[G::TT * 36];
    const uint32_t w = wave_of(p);
    const uint32_t r1 = part_begin(p, w + 1);
    for (uint32_t r = part_begin(p, w); r < r1;) {
        // the piece of group g this range holds: tiles [ta, te)
        const uint32_t g = r / p.T;
        const uint32_t gs = g * p.T;
        const uint32_t te = (r1 < gs + p.T ? r1 : gs + p.T) - gs;
        const uint32_t ta = r - gs;
        const uint32_t b = g / p.gx;
        const RowSetup rs = row_setup(A, D, bias, Dn, lens, L, g - b * p.gx, b);
        const int64_t t_begin = static_cast<int64_t>(ta) * G::TT;
        const int64_t t_end = static_cast<int64_t>(te) * G::TT < L ? static_cast<int64_t>(te) * G::TT : L;
        const uint32_t s_begin = ta > 0 ? wave_holding(p, gs) : w;  // earlier pieces of this group
        const int64_t base = rs.row * L;
        const float* Bb = B + static_cast<int64_t>(b) * kN * L;
        const float* Cb = C + static_cast<int64_t>(b) * kN * L;
        const typename E::storage* zp = z ? z + base : nullptr;
        float h[kN];
        if (__all(rs.pow_ok)) {
            fold_carry<true>(h, rs.A2, agg, h0, s_begin, w, rs.row);
            main_body<E, HAS_Z, SOFTPLUS, true, VARLEN, RAGGED, SAVE>(rs, h, u + base, delta + base, zp, out + base,
                                                                    Bb, Cb, L, srow, sbc, t_begin, t_end, saved, R);
        } else {
            fold_carry<false>(h, rs.A2, agg, h0, s_begin, w, rs.row);
            main_body<E, HAS_Z, SOFTPLUS, false, VARLEN, RAGGED, SAVE>(rs, h, u + base, delta + base, zp, out + base,
                                                                     Bb, Cb, L, srow, sbc, t_begin, t_end, saved, R);
        }
        if (last_state && rs.active && te == p.T) {
            float4* dst = reinterpret_cast<float4*>(last_state + rs.row * kN);
#pragma unroll
            for (int q = 0; q < kN / 4; ++q)
                dst[q] = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
        }
        r = gs + te;
    }
}

// Aggregate of one segment: (sum of delta, end state of the segment started from h = 0).
// POW walks the segment backward (acc_n += x_s B_s R^(n+1), R the product of the later
// Abar_0); the general path runs the recurrence forward without outputs.
template <class E, bool SOFTPLUS, bool POW, bool VARLEN, bool RAGGED>
__device__ __forceinline__ void agg_body(const RowSetup& rs, const typename E::storage* __restrict__ up,
                                         const typename E::storage* __restrict__ dp,
                                         const float* __restrict__ Bb, int64_t L, uint32_t* srow,
                                         float* sbc, int64_t t_begin, int64_t t_end, float (&acc)[kN],
                                         float& dsum) {
    using G = Geo<E>;
    constexpr int TT = G::TT, W = G::W;
    const uint32_t* su = srow;
    const uint32_t* sd = srow + W * 64;
#pragma unroll
    for (int n = 0; n < kN; ++n) acc[n] = 0.0f;
    dsum = 0.0f;
    float Rp = 1.0f;
    RawUD<E> pre;
    RawBC<E> bpre;
    const int64_t ntiles = (t_end - t_begin + TT - 1) / TT;
    // tiles in visiting order (POW: from the last tile of the segment back to the first)
    int64_t t0 = POW ? t_begin + (ntiles - 1) * TT : t_begin;
    load_ud<E, RAGGED>(pre, up, dp, t0, t_end, L);
    load_bc<E, false, RAGGED>(bpre, Bb, nullptr, L, t0, t_end);
    for (int64_t k = 0; k < ntiles; ++k) {
        __syncthreads();
        stage_ud<E>(srow, pre);
        stage_bc<E, false, VARLEN>(sbc, bpre, t0, rs.stop);
        __syncthreads();
        const int64_t tnext = POW ? t0 - TT : t0 + TT;
        if (k + 1 < ntiles) {
            load_ud<E, RAGGED>(pre, up, dp, tnext, t_end, L);
            load_bc<E, false, RAGGED>(bpre, Bb, nullptr, L, tnext, t_end);
        }
        const int nsteps = tile_steps<RAGGED, TT>(t0, t_end);
        if (POW) {
            // The scalars and the B values of the next pair are read one iteration ahead, so an
            // iteration does not start by waiting for its own LDS reads (unrolled by two so the
            // current / next register sets alternate instead of being copied).
            Pair cur = pair_of<E, SOFTPLUS, true, false, VARLEN>(su, sd, nsteps - 2, rs, t0);
            BPair bcur = b_pair(sbc, nsteps - 2);
#pragma unroll 2
            for (int j = nsteps - 2; j >= 0; j -= 2) {
                const int jn = j >= 2 ? j - 2 : 0;
                const Pair nxt = pair_of<E, SOFTPLUS, true, false, VARLEN>(su, sd, jn, rs, t0);
                const BPair bnxt = b_pair(sbc, jn);
                // step j + 1 first (backward), then step j
                const float R1 = Rp;
                const float R0 = Rp * cur.a[1];
                Rp = R0 * cur.a[0];
                float w1 = cur.x[1], w0 = cur.x[0];
#pragma unroll
                for (int n = 0; n < kN; ++n) {
                    w1 *= R1;
                    w0 *= R0;
                    acc[n] = fmaf(bcur.b[1][n], w1, acc[n]);
                    acc[n] = fmaf(bcur.b[0][n], w0, acc[n]);
                }
                dsum += cur.d[1] + cur.d[0];
                cur = nxt;
                bcur = bnxt;
            }
        } else {
#pragma unroll 1
            for (int j = 0; j < nsteps; j += 2) {
                float u0, u1, r0, r1;
                staged2<E>(su, j, u0, u1);
                staged2<E>(sd, j, r0, r1);
                const float4* b0 = reinterpret_cast<const float4*>(sbc + j * 20);
                const float4* b1 = reinterpret_cast<const float4*>(sbc + (j + 1) * 20);
                const float d0 = (VARLEN && t0 + j >= rs.stop) ? 0.0f : delta_of<SOFTPLUS>(r0, rs.bias);
                const float d1 = (VARLEN && t0 + j + 1 >= rs.stop) ? 0.0f : delta_of<SOFTPLUS>(r1, rs.bias);
                const float x0 = (VARLEN && t0 + j >= rs.stop) ? 0.0f : d0 * u0;
                const float x1 = (VARLEN && t0 + j + 1 >= rs.stop) ? 0.0f : d1 * u1;
#pragma unroll
                for (int q = 0; q < kN / 4; ++q) {
                    const float4 y0 = b0[q], y1 = b1[q];
                    const float c0[4] = {y0.x, y0.y, y0.z, y0.w};
                    const float c1[4] = {y1.x, y1.y, y1.z, y1.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int n = 4 * q + i;
                        acc[n] = fmaf(fast_exp2(d0 * rs.A2[n]), acc[n], x0 * c0[i]);
                        acc[n] = fmaf(fast_exp2(d1 * rs.A2[n]), acc[n], x1 * c1[i]);
                    }
                }
                dsum += d0 + d1;
            }
        }
        t0 = tnext;
    }
}

// Wavefront w's aggregate: the last piece of its range, unless that piece ends its group (then
// nothing later in the group needs it and the wavefront has no aggregate to compute).
template <class E, bool SOFTPLUS, bool VARLEN, bool RAGGED>
__global__ __launch_bounds__(64) void scan_agg_kernel(
    const typename E::storage* __restrict__ u, const typename E::storage* __restrict__ delta,
    const float* __restrict__ A, const float* __restrict__ B, const float* __restrict__ bias,
    float* __restrict__ agg, const int32_t* __restrict__ lens, int64_t Dn, int64_t L, Part p) {
    using G = Geo<E>;
    __shared__ uint32_t srow[G::kRowWords];
    __shared__ __align__(16) float sbc[G::TT * 20];
    const uint32_t w = wave_of(p);
    const uint32_t r0 = part_begin(p, w), r1 = part_begin(p, w + 1);
    const uint32_t g = (r1 - 1) / p.T;
    const uint32_t gs = g * p.T;
    const uint32_t te = r1 - gs;
    if (r1 <= r0 || te == p.T) return;  // uniform over the wavefront
    const uint32_t ta = (r0 > gs ? r0 : gs) - gs;
    const uint32_t b = g / p.gx;
    const RowSetup rs = row_setup(A, nullptr, bias, Dn, lens, L, g - b * p.gx, b);
    const int64_t t_begin = static_cast<int64_t>(ta) * G::TT;
    const int64_t t_end = static_cast<int64_t>(te) * G::TT;  // < L: the piece does not end the group
    const int64_t base = rs.row * L;
    const float* Bb = B + static_cast<int64_t>(b) * kN * L;
    float acc[kN], dsum;
    if (__all(rs.pow_ok))
        agg_body<E, SOFTPLUS, true, VARLEN, RAGGED>(rs, u + base, delta + base, Bb, L, srow, sbc, t_begin, t_end, acc,
                                                    dsum);
    else
        agg_body<E, SOFTPLUS, false, VARLEN, RAGGED>(rs, u + base, delta + base, Bb, L, srow, sbc, t_begin, t_end, acc,
                                                     dsum);
    // every lane stores (inactive lanes hold a copy of the group's last channel, never read for
    // an output): the slot is dense
    float* a = agg + static_cast<size_t>(w) * (kN + 1) * 64 + threadIdx.x;
#pragma unroll
    for (int n = 0; n < kN; ++n) a[n * 64] = acc[n];
    a[kN * 64] = dsum;
}

template <class E, bool HAS_Z, bool SOFTPLUS, bool VARLEN, bool RAGGED>
hipError_t launch_fast_t(const ScanLaunch& a, const ScanPlan& pl, float* ws, hipStream_t stream) {
    using S_t = typename E::storage;
    float* agg = ws;
    const dim3 block(64);
    const int64_t gx = (a.Dn + 63) / 64;
    const int64_t T = (a.L + Geo<E>::TT - 1) / Geo<E>::TT;
    const int64_t GT = a.Bt * gx * T;  // < 2^32 (plan_fast refuses larger)
    Part p;
    p.T = static_cast<uint32_t>(T);
    p.W = static_cast<uint32_t>(pl.waves);
    p.q = static_cast<uint32_t>(GT / pl.waves);
    p.rem = static_cast<uint32_t>(GT % pl.waves);
    p.gx = static_cast<uint32_t>(gx);
    p.X = static_cast<uint32_t>(pl.xcds);
    p.xq = p.W / p.X;
    p.xr = p.W % p.X;
    const int64_t R = a.Bt * a.Dn;
    const dim3 grid(static_cast<unsigned>(p.W));
    mark(a, 0, stream);
    if (pl.segments > 1)
        scan_agg_kernel<E, SOFTPLUS, VARLEN, RAGGED><<<grid, block, 0, stream>>>(
            static_cast<const S_t*>(a.u), static_cast<const S_t*>(a.delta), a.A, a.B, a.bias, agg, a.lens, a.Dn,
            a.L, p);
    mark(a, 1, stream);
    if (a.saved)
        scan_main_kernel<E, HAS_Z, SOFTPLUS, VARLEN, RAGGED, true><<<grid, block, 0, stream>>>(
            static_cast<const S_t*>(a.u), static_cast<const S_t*>(a.delta), static_cast<const S_t*>(a.z), a.A, a.B,
            a.C, a.D, a.bias, agg, a.h0, static_cast<S_t*>(a.out), a.last_state, a.lens, a.saved, a.Dn, a.L, R, p);
    else
        scan_main_kernel<E, HAS_Z, SOFTPLUS, VARLEN, RAGGED, false><<<grid, block, 0, stream>>>(
            static_cast<const S_t*>(a.u), static_cast<const S_t*>(a.delta), static_cast<const S_t*>(a.z), a.A, a.B,
            a.C, a.D, a.bias, agg, a.h0, static_cast<S_t*>(a.out), a.last_state, a.lens, nullptr, a.Dn, a.L, R, p);
    mark(a, 2, stream);
    return hipGetLastError();
}

template <class E, bool VARLEN, bool RAGGED>
hipError_t launch_fast_v(const ScanLaunch& a, const ScanPlan& p, float* ws, hipStream_t stream) {
    const bool hz = a.z != nullptr;
    if (a.softplus)
        return hz ? launch_fast_t<E, true, true, VARLEN, RAGGED>(a, p, ws, stream)
                  : launch_fast_t<E, false, true, VARLEN, RAGGED>(a, p, ws, stream);
    return hz ? launch_fast_t<E, true, false, VARLEN, RAGGED>(a, p, ws, stream)
              : launch_fast_t<E, false, false, VARLEN, RAGGED>(a, p, ws, stream);
}

// Rows of any length (not whole 16-byte vectors) run the same kernels with element-aligned
// loads and stores and the steps past L masked as with per-batch lengths.
template <class E>
hipError_t launch_fast_e(const ScanLaunch& a, const ScanPlan& p, float* ws, hipStream_t stream) {
    if (!a.vec_ok) return launch_fast_v<E, true, true>(a, p, ws, stream);
    return a.lens ? launch_fast_v<E, true, false>(a, p, ws, stream) : launch_fast_v<E, false, false>(a, p, ws, stream);
}

}  // namespace

// Wavefronts: two per SIMD for bf16 rows and one for fp32 rows, all resident at once (the main
// kernel is built for two per SIMD: 256 VGPRs, no spills).  More were slower: Mamba-2.8B layer
// 226 us at two per SIMD, 259 us at three, 239 / 250 us at 1.9 / 2.25 (uneven SIMD loads);
// Mamba-130M fp32 layer 203 us at one per SIMD, 218 us at 1.5, 233 us at 2; long context 1341 us at
// one, 1359 at 1.5 -- more streams in flight evict more of each other's lines.  At least two tiles
// each (a shorter piece spends more on folding the aggregates before it than it saves), except on
// short rows.  fp32 tiles are whole 128-byte lines (long context 1.45 -> 1.29 ms against 64-byte
// tiles, which fetched every line twice).  `waves_override` > 0 replaces the count (tests use it to force many or few
// pieces per group, and ranges that cross groups).  `segments` reports whether some range ends
// inside a group, i.e. whether the aggregate kernel has work.
ScanPlan plan_fast(const ScanLaunch& a, int num_cus, int64_t waves_override) {
    ScanPlan p;
    const int TT = fast_tile_bytes(a.bf16) / (a.bf16 ? 2 : 4);
    const int64_t groups = a.Bt * ((a.Dn + 63) / 64);
    const int64_t tiles = (a.L + TT - 1) / TT;
    const int64_t GT = groups * tiles;
    int64_t W = (a.bf16 ? 8LL : 4LL) * (num_cus > 0 ? num_cus : 256);
    // pieces of at least two tiles, unless the rows are short (under 16 tiles): then parallelism
    // matters more than the fold (2 x 64 x 256 fp32: 33 -> 22 us with one-tile pieces)
    const int64_t min_piece = tiles >= 16 ? 2 : 1;
    if (W > GT / min_piece) W = GT / min_piece;
    if (waves_override > 0) W = waves_override;
    if (W > GT) W = GT;
    if (W > 0x7fffffffLL) W = 0x7fffffffLL;
    if (W < 1) W = 1;
    p.fits = GT < (int64_t{1} << 32);  // the kernels count tiles in 32 bits
    p.waves = W;
    p.xcds = num_cus >= 64 && num_cus % 32 == 0 ? num_cus / 32 : 1;  // 32 CUs per XCD on gfx950
    // every range ends on a group boundary exactly when each wavefront takes whole groups
    const bool whole = W <= groups && groups % W == 0;
    p.segments = whole ? 1 : 2;
    p.seg_len = 0;
    p.workspace_bytes = fast_workspace_bytes(a, p);
    return p;
}

size_t fast_workspace_bytes(const ScanLaunch& a, const ScanPlan& p) {
    (void)a;
    return p.segments > 1 ? static_cast<size_t>(p.waves) * (kN + 1) * 64 * sizeof(float) : 0;
}

hipError_t launch_scan_fast(const ScanLaunch& a, const ScanPlan& p, float* ws, hipStream_t stream) {
    return a.bf16 ? launch_fast_e<BF16>(a, p, ws, stream) : launch_fast_e<F32>(a, p, ws, stream);
}

}  // namespace mss
