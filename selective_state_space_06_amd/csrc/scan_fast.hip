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
//   * u / delta / z stream in as 16-byte vectors of the lane's own row, a 64-byte tile (32 bf16 or
//     16 fp32 steps) at a time; the next tile is prefetched into VGPRs while the current one
//     runs, and the current one sits in a lane-private LDS row that the step loop indexes;
//     outputs overwrite the consumed u slots and leave as 16-byte stores per tile;
//   * B_t and C_t are the same for all 64 lanes of a wave (one batch): a kernel first writes a
//     time-major copy (Bt, L, 32) of B and C; each tile's block of it is prefetched with
//     coalesced 16-byte loads together with the u / delta / z tile, written to LDS at the tile
//     boundary, and read back per step as broadcast 16-byte LDS loads (all lanes one address);
//   * long sequences are split into S segments per channel group.  A first kernel computes,
//     per segment, the pair (sum of delta, local end state from h = 0); the main kernel folds
//     the pairs of the preceding segments with the associative operator
//     (a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2) into its starting state and runs the segment.
//
// exp is exp2 of a log2(e)-prescaled argument.  When every row of a wave satisfies
// A[d, n] == (n + 1) A[d, 0] exactly (the S4D-real A = -(1..N) of the tutorial's init),
// Abar_n = Abar_0^(n+1) is formed by repeated multiplication (one exp2 per (b, d, t)); the
// aggregate pass then uses the backward form sum_s x_s B_s R_s^(n+1), R_s the product of the
// later Abar_0, which costs two VALU operations per state update.
#include "device_math.hpp"
#include "mss_internal.hpp"

namespace mss {
namespace {

constexpr int kBCW = 2 * kN;                   // B|C floats per time step in the time-major copy
constexpr int kNV = kFastTileBytes / 16;       // 16-byte vectors per row and array in a tile
constexpr int kRowWords = kFastTileBytes / 4 + 1;  // LDS words per lane row (+1: bank skew)

// (Bt, N, L) B and C -> (Bt, L, 2N): B in [0, N), C in [N, 2N).
__global__ __launch_bounds__(256) void bc_transpose_kernel(const float* __restrict__ B,
                                                           const float* __restrict__ C,
                                                           float* __restrict__ bc, int64_t L,
                                                           int64_t total) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = i / L, t = i - b * L;
        const float* Bb = B + b * kN * L + t;
        const float* Cb = C + b * kN * L + t;
        float v[kBCW];
#pragma unroll
        for (int n = 0; n < kN; ++n) {
            v[n] = Bb[n * L];
            v[kN + n] = Cb[n * L];
        }
        float4* dst = reinterpret_cast<float4*>(bc + i * kBCW);
#pragma unroll
        for (int q = 0; q < kBCW / 4; ++q)
            dst[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
}

struct RowSetup {
    int64_t row;      // flat (b, d) row, clamped to a valid row for inactive lanes
    bool active;      // lane maps to a real channel
    float A2[kN];     // A[d, n] * log2(e)
    float bias, dskip;
    bool pow_ok;
};

__device__ __forceinline__ RowSetup row_setup(const float* __restrict__ A, const float* __restrict__ D,
                                              const float* __restrict__ bias, int64_t Dn) {
    RowSetup r;
    const int64_t d = (int64_t)blockIdx.x * 64 + threadIdx.x;
    r.active = d < Dn;
    const int64_t dc = r.active ? d : Dn - 1;
    r.row = (int64_t)blockIdx.y * Dn + dc;
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

// One tile of this lane's row (u, delta and optionally z), as loaded from HBM.
struct Raw {
    uint4 u[kNV], d[kNV], z[kNV];
};

// Loads the tile starting at t0.  Vectors at or past t_end re-read the last valid vector (their
// steps are never used), so every load is unconditional and in bounds.
template <class E, bool HAS_Z>
__device__ __forceinline__ void load_tile(Raw& r, const typename E::storage* __restrict__ up,
                                          const typename E::storage* __restrict__ dp,
                                          const typename E::storage* __restrict__ zp, int64_t t0,
                                          int64_t t_end) {
    constexpr int V = E::kPerVec;
#pragma unroll
    for (int v = 0; v < kNV; ++v) {
        int64_t t = t0 + v * V;
        t = t < t_end ? t : t_end - V;
        r.u[v] = *reinterpret_cast<const uint4*>(up + t);
        r.d[v] = *reinterpret_cast<const uint4*>(dp + t);
        if (HAS_Z) r.z[v] = *reinterpret_cast<const uint4*>(zp + t);
    }
}

// Lane-private LDS rows (kRowWords words per lane and array).
__device__ __forceinline__ void stage_vec(uint32_t* row, int v, const uint4& x) {
    row[4 * v + 0] = x.x;
    row[4 * v + 1] = x.y;
    row[4 * v + 2] = x.z;
    row[4 * v + 3] = x.w;
}

template <bool HAS_Z>
__device__ __forceinline__ void stage_tile(uint32_t* ru, uint32_t* rd, uint32_t* rz, const Raw& r) {
#pragma unroll
    for (int v = 0; v < kNV; ++v) {
        stage_vec(ru, v, r.u[v]);
        stage_vec(rd, v, r.d[v]);
        if (HAS_Z) stage_vec(rz, v, r.z[v]);
    }
}

template <bool SOFTPLUS>
__device__ __forceinline__ float delta_of(float raw, float bias) {
    const float pre = raw + bias;
    return SOFTPLUS ? softplus(pre) : pre;
}

struct BCStep {
    float v[kBCW];
};

// The tile's B|C block from the time-major copy: TT steps x 128 bytes, contiguous; lane l holds
// 16-byte chunks l, l + 64, ...  Steps at or past t_end are clamped to the last valid step.
// (Plain words: an array of vector structs here ends up in scratch memory.)
template <int TT>
struct RawBC {
    static constexpr int kChunks = TT * kBCW / 4 / 64;
    uint32_t w[4 * kChunks];
};

template <int TT>
__device__ __forceinline__ void load_bc_tile(RawBC<TT>& r, const float* __restrict__ bcb, int64_t t0,
                                             int64_t t_end) {
#pragma unroll
    for (int k = 0; k < RawBC<TT>::kChunks; ++k) {
        const int chunk = threadIdx.x + 64 * k;  // 8 chunks per step
        int64_t t = t0 + chunk / 8;
        t = t < t_end ? t : t_end - 1;
        const uint4 v = *reinterpret_cast<const uint4*>(bcb + t * kBCW + (chunk % 8) * 4);
        r.w[4 * k] = v.x; r.w[4 * k + 1] = v.y; r.w[4 * k + 2] = v.z; r.w[4 * k + 3] = v.w;
    }
}

template <int TT>
__device__ __forceinline__ void stage_bc_tile(float* sbc, const RawBC<TT>& r) {
#pragma unroll
    for (int k = 0; k < RawBC<TT>::kChunks; ++k)
        reinterpret_cast<uint4*>(sbc)[threadIdx.x + 64 * k] =
            make_uint4(r.w[4 * k], r.w[4 * k + 1], r.w[4 * k + 2], r.w[4 * k + 3]);
}

// Broadcast read of B_t | C_t from the LDS block: every lane reads the same 128 bytes.
__device__ __forceinline__ BCStep read_bc(const float* sbc_t) {
    BCStep r;
#pragma unroll
    for (int q = 0; q < kBCW / 4; ++q) {
        const float4 v = reinterpret_cast<const float4*>(sbc_t)[q];
        r.v[4 * q] = v.x; r.v[4 * q + 1] = v.y; r.v[4 * q + 2] = v.z; r.v[4 * q + 3] = v.w;
    }
    return r;
}

// One time step for one lane: 16 state updates and y = C.h.
template <bool POW>
__device__ __forceinline__ float step_main(float (&h)[kN], const float (&A2)[kN], float dl, float x,
                                           const BCStep& bc) {
    float y0 = 0.0f, y1 = 0.0f;
    if (POW) {
        const float a = fast_exp2(dl * A2[0]);
        float p = a;
#pragma unroll
        for (int n = 0; n < kN; ++n) {
            if (n) p *= a;
            h[n] = fmaf(p, h[n], x * bc.v[n]);
            if (n & 1) y1 = fmaf(bc.v[kN + n], h[n], y1);
            else y0 = fmaf(bc.v[kN + n], h[n], y0);
        }
    } else {
#pragma unroll
        for (int n = 0; n < kN; ++n) {
            h[n] = fmaf(fast_exp2(dl * A2[n]), h[n], x * bc.v[n]);
            if (n & 1) y1 = fmaf(bc.v[kN + n], h[n], y1);
            else y0 = fmaf(bc.v[kN + n], h[n], y0);
        }
    }
    return y0 + y1;
}

// Element i of the staged row (bf16: two per word, fp32: one per word).
template <class E>
__device__ __forceinline__ float staged(const uint32_t* row, int i) {
    if (E::kPerVec == 8) {
        const uint32_t w = row[i >> 1];
        return (i & 1) ? bf16_hi(w) : bf16_lo(w);
    }
    return __uint_as_float(row[i]);
}

// Outputs i and i + 1 (i even) written over the consumed u slots.
template <class E>
__device__ __forceinline__ void put_out2(uint32_t* row, int i, float o0, float o1) {
    if (E::kPerVec == 8) {
        row[i >> 1] = pack_bf16x2(o0, o1);
    } else {
        row[i] = __float_as_uint(o0);
        row[i + 1] = __float_as_uint(o1);
    }
}

template <class E, bool HAS_Z, bool SOFTPLUS, bool POW>
__device__ __forceinline__ void main_body(
    const RowSetup& rs, float (&h)[kN], const typename E::storage* __restrict__ up,
    const typename E::storage* __restrict__ dp, const typename E::storage* __restrict__ zp,
    typename E::storage* __restrict__ op, const float* __restrict__ bcb, uint32_t* ru, uint32_t* rd,
    uint32_t* rz, float* sbc, int64_t t_begin, int64_t t_end) {
    constexpr int V = E::kPerVec;
    constexpr int TT = kNV * V;
    Raw pre;
    RawBC<TT> bpre;
    load_tile<E, HAS_Z>(pre, up, dp, zp, t_begin, t_end);
    load_bc_tile<TT>(bpre, bcb, t_begin, t_end);
    for (int64_t t0 = t_begin; t0 < t_end; t0 += TT) {
        stage_tile<HAS_Z>(ru, rd, rz, pre);
        stage_bc_tile<TT>(sbc, bpre);
        if (t0 + TT < t_end) {
            load_tile<E, HAS_Z>(pre, up, dp, zp, t0 + TT, t_end);
            load_bc_tile<TT>(bpre, bcb, t0 + TT, t_end);
        }
        const int nsteps = static_cast<int>(t_end - t0 < TT ? t_end - t0 : TT);  // even
#pragma unroll 1
        for (int j = 0; j < nsteps; j += 2) {
            const float u0 = staged<E>(ru, j), u1 = staged<E>(ru, j + 1);
            const float d0 = delta_of<SOFTPLUS>(staged<E>(rd, j), rs.bias);
            const float y0 = step_main<POW>(h, rs.A2, d0, d0 * u0, read_bc(sbc + j * kBCW));
            const float d1 = delta_of<SOFTPLUS>(staged<E>(rd, j + 1), rs.bias);
            const float y1 = step_main<POW>(h, rs.A2, d1, d1 * u1, read_bc(sbc + (j + 1) * kBCW));
            float o0 = fmaf(rs.dskip, u0, y0), o1 = fmaf(rs.dskip, u1, y1);
            if (HAS_Z) {
                o0 *= silu(staged<E>(rz, j));
                o1 *= silu(staged<E>(rz, j + 1));
            }
            put_out2<E>(ru, j, o0, o1);
        }
        if (rs.active) {
#pragma unroll
            for (int v = 0; v < kNV; ++v)
                if (t0 + v * V < t_end)
                    *reinterpret_cast<uint4*>(op + t0 + v * V) =
                        make_uint4(ru[4 * v], ru[4 * v + 1], ru[4 * v + 2], ru[4 * v + 3]);
        }
    }
}

// Folds the aggregates of segments [0, seg) into the starting state of segment seg.
template <bool POW>
__device__ __forceinline__ void fold_carry(float (&h)[kN], const float (&A2)[kN],
                                           const float* __restrict__ agg, int seg, int64_t R,
                                           int64_t row) {
#pragma unroll
    for (int n = 0; n < kN; ++n) h[n] = 0.0f;
    for (int s = 0; s < seg; ++s) {
        const float* a = agg + (int64_t)s * (kN + 1) * R + row;
        const float sd = a[(int64_t)kN * R];
        if (POW) {
            const float q = fast_exp2(sd * A2[0]);
            float p = q;
#pragma unroll
            for (int n = 0; n < kN; ++n) {
                if (n) p *= q;
                h[n] = fmaf(p, h[n], a[(int64_t)n * R]);
            }
        } else {
#pragma unroll
            for (int n = 0; n < kN; ++n) h[n] = fmaf(fast_exp2(sd * A2[n]), h[n], a[(int64_t)n * R]);
        }
    }
}

template <class E, bool HAS_Z, bool SOFTPLUS>
__global__ __launch_bounds__(64) void scan_main_kernel(
    const typename E::storage* __restrict__ u, const typename E::storage* __restrict__ delta,
    const typename E::storage* __restrict__ z, const float* __restrict__ A,
    const float* __restrict__ bc, const float* __restrict__ D, const float* __restrict__ bias,
    const float* __restrict__ agg, typename E::storage* __restrict__ out,
    float* __restrict__ last_state, int64_t Dn, int64_t L, int64_t seg_len, int S) {
    constexpr int TT = kNV * E::kPerVec;
    __shared__ uint32_t rows[3 * 64 * kRowWords];
    __shared__ __align__(16) float sbc[TT * kBCW];
    uint32_t* ru = rows + threadIdx.x * kRowWords;
    uint32_t* rd = ru + 64 * kRowWords;
    uint32_t* rz = rd + 64 * kRowWords;
    const RowSetup rs = row_setup(A, D, bias, Dn);
    const int seg = blockIdx.z;
    const int64_t R = (int64_t)gridDim.y * Dn;
    const int64_t t_begin = (int64_t)seg * seg_len;
    const int64_t t_end = (t_begin + seg_len < L) ? t_begin + seg_len : L;
    const int64_t base = rs.row * L;
    const float* bcb = bc + (int64_t)blockIdx.y * L * kBCW;
    const typename E::storage* zp = z ? z + base : nullptr;
    float h[kN];
    if (__all(rs.pow_ok)) {
        fold_carry<true>(h, rs.A2, agg, seg, R, rs.row);
        main_body<E, HAS_Z, SOFTPLUS, true>(rs, h, u + base, delta + base, zp, out + base, bcb, ru, rd,
                                            rz, sbc, t_begin, t_end);
    } else {
        fold_carry<false>(h, rs.A2, agg, seg, R, rs.row);
        main_body<E, HAS_Z, SOFTPLUS, false>(rs, h, u + base, delta + base, zp, out + base, bcb, ru, rd,
                                             rz, sbc, t_begin, t_end);
    }
    if (last_state && rs.active && seg == S - 1) {
        float4* dst = reinterpret_cast<float4*>(last_state + rs.row * kN);
#pragma unroll
        for (int q = 0; q < kN / 4; ++q)
            dst[q] = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
    }
}

// Aggregate of one segment: (sum of delta, end state of the segment started from h = 0).
// POW walks the segment backward (acc_n += x_s B_s R^(n+1), R the product of the later
// Abar_0); the general path runs the recurrence forward without outputs.
template <class E, bool SOFTPLUS, bool POW>
__device__ __forceinline__ void agg_body(const RowSetup& rs, const typename E::storage* __restrict__ up,
                                         const typename E::storage* __restrict__ dp,
                                         const float* __restrict__ bcb, uint32_t* ru, uint32_t* rd,
                                         float* sbc, int64_t t_begin, int64_t t_end, float (&acc)[kN],
                                         float& dsum) {
    constexpr int V = E::kPerVec;
    constexpr int TT = kNV * V;
#pragma unroll
    for (int n = 0; n < kN; ++n) acc[n] = 0.0f;
    dsum = 0.0f;
    float Rp = 1.0f;
    Raw pre;
    RawBC<TT> bpre;
    const int64_t ntiles = (t_end - t_begin + TT - 1) / TT;
    // tiles in visiting order (POW: from the last tile of the segment back to the first)
    int64_t t0 = POW ? t_begin + (ntiles - 1) * TT : t_begin;
    load_tile<E, false>(pre, up, dp, nullptr, t0, t_end);
    load_bc_tile<TT>(bpre, bcb, t0, t_end);
    for (int64_t k = 0; k < ntiles; ++k) {
        stage_tile<false>(ru, rd, nullptr, pre);
        stage_bc_tile<TT>(sbc, bpre);
        const int64_t tnext = POW ? t0 - TT : t0 + TT;
        if (k + 1 < ntiles) {
            load_tile<E, false>(pre, up, dp, nullptr, tnext, t_end);
            load_bc_tile<TT>(bpre, bcb, tnext, t_end);
        }
        const int nsteps = static_cast<int>(t_end - t0 < TT ? t_end - t0 : TT);
        if (POW) {
#pragma unroll 1
            for (int j = nsteps - 1; j >= 0; --j) {
                const float* bt = sbc + j * kBCW;
                const float dl = delta_of<SOFTPLUS>(staged<E>(rd, j), rs.bias);
                float w = dl * staged<E>(ru, j) * Rp;
#pragma unroll
                for (int q = 0; q < kN / 4; ++q) {
                    const float4 b4 = reinterpret_cast<const float4*>(bt)[q];
                    const float bq[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (q | i) w *= Rp;
                        acc[4 * q + i] = fmaf(bq[i], w, acc[4 * q + i]);
                    }
                }
                Rp *= fast_exp2(dl * rs.A2[0]);
                dsum += dl;
            }
        } else {
#pragma unroll 1
            for (int j = 0; j < nsteps; ++j) {
                const float* bt = sbc + j * kBCW;
                const float dl = delta_of<SOFTPLUS>(staged<E>(rd, j), rs.bias);
                const float x = dl * staged<E>(ru, j);
#pragma unroll
                for (int q = 0; q < kN / 4; ++q) {
                    const float4 b4 = reinterpret_cast<const float4*>(bt)[q];
                    const float bq[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[4 * q + i] = fmaf(fast_exp2(dl * rs.A2[4 * q + i]), acc[4 * q + i], x * bq[i]);
                }
                dsum += dl;
            }
        }
        t0 = tnext;
    }
}

template <class E, bool SOFTPLUS>
__global__ __launch_bounds__(64) void scan_agg_kernel(
    const typename E::storage* __restrict__ u, const typename E::storage* __restrict__ delta,
    const float* __restrict__ A, const float* __restrict__ bc, const float* __restrict__ bias,
    float* __restrict__ agg, int64_t Dn, int64_t L, int64_t seg_len) {
    constexpr int TT = kNV * E::kPerVec;
    __shared__ uint32_t rows[2 * 64 * kRowWords];
    __shared__ __align__(16) float sbc[TT * kBCW];
    uint32_t* ru = rows + threadIdx.x * kRowWords;
    uint32_t* rd = ru + 64 * kRowWords;
    const RowSetup rs = row_setup(A, nullptr, bias, Dn);
    const int seg = blockIdx.z;
    const int64_t R = (int64_t)gridDim.y * Dn;
    const int64_t t_begin = (int64_t)seg * seg_len;
    const int64_t t_end = (t_begin + seg_len < L) ? t_begin + seg_len : L;
    const int64_t base = rs.row * L;
    const float* bcb = bc + (int64_t)blockIdx.y * L * kBCW;
    float acc[kN], dsum;
    if (__all(rs.pow_ok))
        agg_body<E, SOFTPLUS, true>(rs, u + base, delta + base, bcb, ru, rd, sbc, t_begin, t_end, acc, dsum);
    else
        agg_body<E, SOFTPLUS, false>(rs, u + base, delta + base, bcb, ru, rd, sbc, t_begin, t_end, acc, dsum);
    if (rs.active) {
        float* a = agg + (int64_t)seg * (kN + 1) * R + rs.row;
#pragma unroll
        for (int n = 0; n < kN; ++n) a[(int64_t)n * R] = acc[n];
        a[(int64_t)kN * R] = dsum;
    }
}

template <class E, bool HAS_Z, bool SOFTPLUS>
hipError_t launch_fast_t(const ScanLaunch& a, const ScanPlan& p, float* ws, hipStream_t stream) {
    using S_t = typename E::storage;
    float* bc = ws;
    float* agg = ws + a.Bt * a.L * kBCW;
    {
        const int64_t total = a.Bt * a.L;
        int64_t blocks = (total + 255) / 256;
        if (blocks > 65535) blocks = 65535;
        bc_transpose_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(a.B, a.C, bc, a.L, total);
    }
    const dim3 block(64);
    const unsigned gx = static_cast<unsigned>((a.Dn + 63) / 64);
    if (p.segments > 1)
        scan_agg_kernel<E, SOFTPLUS><<<dim3(gx, (unsigned)a.Bt, (unsigned)(p.segments - 1)), block, 0, stream>>>(
            static_cast<const S_t*>(a.u), static_cast<const S_t*>(a.delta), a.A, bc, a.bias, agg, a.Dn,
            a.L, p.seg_len);
    scan_main_kernel<E, HAS_Z, SOFTPLUS><<<dim3(gx, (unsigned)a.Bt, (unsigned)p.segments), block, 0, stream>>>(
        static_cast<const S_t*>(a.u), static_cast<const S_t*>(a.delta), static_cast<const S_t*>(a.z), a.A,
        bc, a.D, a.bias, agg, static_cast<S_t*>(a.out), a.last_state, a.Dn, a.L, p.seg_len, p.segments);
    return hipGetLastError();
}

template <class E>
hipError_t launch_fast_e(const ScanLaunch& a, const ScanPlan& p, float* ws, hipStream_t stream) {
    const bool hz = a.z != nullptr;
    if (a.softplus) return hz ? launch_fast_t<E, true, true>(a, p, ws, stream) : launch_fast_t<E, false, true>(a, p, ws, stream);
    return hz ? launch_fast_t<E, true, false>(a, p, ws, stream) : launch_fast_t<E, false, false>(a, p, ws, stream);
}

}  // namespace

size_t fast_workspace_bytes(const ScanLaunch& a, int segments) {
    return (static_cast<size_t>(a.Bt * a.L) * kBCW +
            static_cast<size_t>(segments > 1 ? segments - 1 : 0) * (kN + 1) * static_cast<size_t>(a.Bt * a.Dn)) *
           sizeof(float);
}

hipError_t launch_scan_fast(const ScanLaunch& a, const ScanPlan& p, float* ws, hipStream_t stream) {
    return a.bf16 ? launch_fast_e<BF16>(a, p, ws, stream) : launch_fast_e<F32>(a, p, ws, stream);
}

}  // namespace mss
