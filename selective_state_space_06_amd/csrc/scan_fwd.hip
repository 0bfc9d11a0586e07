// scan_fwd.hip -- forward selective scan (S6) for gfx950.
//
// Computes, per batch b, channel d and state n (Mamba paper Section 3 / Algorithm 2, as
// coded on the Keras/TensorFlow Mamba tutorial page in `selective_scan` and
// `MambaBlock.ssm`; the upstream mamba README's "Selective SSM" layer):
//   delta_t = softplus(delta_raw_t + bias_d)   Abar = exp(delta_t A_dn)
//   h_t = Abar h_{t-1} + delta_t B_nt u_t (h_0 = 0, or a given state)
//   out_t = (sum_n C_nt h_t + D_d u_t) silu(z_t)
//
// Work decomposition, for d_state N = 16, 32, 64 or 128:
//   * a lane owns SPL states of one channel (row b, d) in VGPRs, sequential in t (SPL = 8 at
//     d_state 32 and 64, 16 otherwise): Q = N / SPL neighbouring lanes share a channel, so a
//     wave holds 64 / Q consecutive channels of one batch; each lane's part of C.h meets its
//     neighbours' through DPP adds;
//   * B_t and C_t are the same for every channel of a batch: they are staged once per time tile
//     in LDS, transposed to [t][n], shared by the workgroup's wavefronts (one at d_state 16, four
//     otherwise), and read back as broadcast 16-byte LDS loads;
//   * u / delta / z / out move between HBM and LDS in 16-byte vectors along L (coalesced),
//     and the per-element work (bias + softplus, delta * u, the D skip and the silu gate) is
//     done in that coalesced layout, once per element;
//   * long sequences are cut into `S` segments per channel group (grid z) so that enough
//     wavefronts exist to fill the 1024 SIMDs.  An aggregate pass computes, per segment, the
//     pair (sum of delta, local end state from h = 0); a combine pass folds the pairs with
//     the associative operator (a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2) -- the parallel
//     associative scan the tutorial page and the mamba-jax README describe -- into each
//     segment's starting state; the main pass then runs every segment from its true start.
//     A given starting state h0 enters only through segment 0 and the start of that fold; with
//     per-batch sequence lengths, steps at or past a batch's length are identity steps with zero
//     outputs.
//
// exp(delta A) = exp2(delta * A log2e) with A log2e formed once per (d, n).  When a row
// satisfies A[d, n] == (n + 1) A[d, 0] exactly (the S4D-real initialisation A = -(1..N) the
// tutorial uses), Abar_n = Abar_0^(n+1) is formed by repeated multiplication: a lane holding
// states SPL k .. SPL k + SPL - 1 takes exp(delta A[d, SPL k]) and steps it by Abar_0, two exp2
// per (b, d, t) and lane (one when N = 16) instead of SPL.  The choice is made per wavefront on
// the device from the A rows it loads; any other A takes the general path.
#include "device_math.hpp"
#include "mss_internal.hpp"

namespace mss {
namespace {

constexpr int kMain = 0;  // full pass: writes out (and last_state)
constexpr int kAgg = 1;   // aggregate pass: writes (local end state, sum delta) per segment

struct KArgs {
    const void* u;
    const void* delta;
    const void* z;
    const float* A;
    const float* B;
    const float* C;
    const float* D;
    const float* bias;
    void* out;
    float* last_state;
    const float* h0;      // nullable starting state, (rows_total, N)
    const int32_t* lens;  // nullable per-batch sequence lengths
    float* ws;            // [S][N + 1][rows_total] carry workspace
    int64_t Dn, L, seg_len, rows_total;
    int S;
    int N;                // d_state
    int softplus;
};

// Shape of the work for d_state N: SPL states per lane, Q lanes per channel, CH channels per
// wavefront, TT-step tiles, WPB wavefronts per workgroup.  From d_state 32 on, four wavefronts
// (consecutive channel groups of one batch) share each tile's B | C in LDS: a quarter of the
// staging each, and a quarter of the LDS, which leaves room for three wavefronts per SIMD.  Eight
// states per lane at d_state 32 and 64 give twice the wavefronts of sixteen (2560 on the 2.8B
// layer shape at 64, which three per SIMD hold at once, against 1280 that leave a quarter of
// the SIMDs with two and the rest with one).
template <int N>
struct Shape {
    static_assert(N == 16 || N == 32 || N == 64 || N == 128, "d_state");
    static constexpr int SPL = (N == 32 || N == 64) ? 8 : 16;  // states per lane
    static constexpr int Q = N / SPL;
    static constexpr int CH = kRows / Q;
    static constexpr int TT = 32;
    static constexpr int WPB = N >= 32 ? 4 : 1;
};

// Word of entry m of a step's B | C row in LDS (m = n for B_n, N + n for C_n): four pad words
// after every 64, so that the Q blocks of SPL states a wavefront reads at one step (one per lane
// group, 16-byte reads) fall in distinct groups of four banks of the 64.
__host__ __device__ constexpr int bc_word(int m) { return m + 4 * (m / 64); }

template <int N>
struct Smem {
    static constexpr int CH = Shape<N>::CH;
    static constexpr int TT = Shape<N>::TT;
    static constexpr int kRowStride = TT + 4;   // 16-byte pad: lane-row 16 B reads hit distinct banks
    static constexpr int kBCStride = bc_word(2 * N) + 4;
    struct Wave {                  // one wavefront's channels
        float dl[CH][kRowStride];  // delta (phase A) then y (phase B)
        float x[CH][kRowStride];   // delta * u
        float bias[CH];
        float dsk[CH];
    };
    Wave w[Shape<N>::WPB];
    float bc[TT][kBCStride];       // B[0..N-1] | C[0..N-1] per time step, at bc_word positions (shared)
};

// One time step of one lane: its SPL state updates and (main pass) their part of C.h.  A2 holds
// A log2e of the lane's states and A2b that of the channel's state 0; bc points at the step's B
// entries for the lane's states, bc + cofs at its C entries.
template <bool POW, bool WANT_Y, int Q, int SPL>
__device__ __forceinline__ float step_lane(float (&h)[SPL], const float (&A2)[SPL], float A2b, float dl, float x,
                                        const float* __restrict__ bc, int cofs) {
    float Bv[SPL], Cv[SPL];
#pragma unroll
    for (int q = 0; q < SPL / 4; ++q) {
        const float4 b4 = reinterpret_cast<const float4*>(bc)[q];
        Bv[4 * q] = b4.x; Bv[4 * q + 1] = b4.y; Bv[4 * q + 2] = b4.z; Bv[4 * q + 3] = b4.w;
        if (WANT_Y) {
            const float4 c4 = reinterpret_cast<const float4*>(bc + cofs)[q];
            Cv[4 * q] = c4.x; Cv[4 * q + 1] = c4.y; Cv[4 * q + 2] = c4.z; Cv[4 * q + 3] = c4.w;
        }
    }
    float y = 0.0f;
    if (POW) {
        // Abar_n = exp(dl A[d, SPL k]) Abar_0^(n - SPL k) across the lane's states from SPL k
        const float a = fast_exp2(dl * A2b);
        float p = Q == 1 ? a : fast_exp2(dl * A2[0]);
#pragma unroll
        for (int n = 0; n < SPL; ++n) {
            if (n) p *= a;
            h[n] = fmaf(p, h[n], x * Bv[n]);
            if (WANT_Y) y = n ? fmaf(Cv[n], h[n], y) : Cv[0] * h[0];
        }
    } else {
#pragma unroll
        for (int n = 0; n < SPL; ++n) {
            h[n] = fmaf(fast_exp2(dl * A2[n]), h[n], x * Bv[n]);
            if (WANT_Y) y = n ? fmaf(Cv[n], h[n], y) : Cv[0] * h[0];
        }
    }
    return y;
}

// The power path at 16 states per lane keeps each lane's states scaled, g = h / sc with sc the
// scale of the step last taken: step t takes s_t = step_scale(x_t) = x_t + copysign(2^-40, x_t) and
// computes g = (sc / s_t) abar^(n+1) g + B_t, so B enters the state update without a
// multiplication by x (16 fewer per lane and step, against a reciprocal and three more
// multiplications), and the caller scales the channel's C.g by s_t.  Adding s_t B_t for x_t B_t
// moves each state by at most 2^-40 |B_t| per step (B is staged as 0 past a sequence's end).

template <bool WANT_Y, int Q, int SPL>
__device__ __forceinline__ float step_lane_scaled(float (&g)[SPL], const float (&A2)[SPL], float A2b, float dl,
                                                  float r, const float* __restrict__ bc, int cofs) {
    float Bv[SPL], Cv[SPL];
#pragma unroll
    for (int q = 0; q < SPL / 4; ++q) {
        const float4 b4 = reinterpret_cast<const float4*>(bc)[q];
        Bv[4 * q] = b4.x; Bv[4 * q + 1] = b4.y; Bv[4 * q + 2] = b4.z; Bv[4 * q + 3] = b4.w;
        if (WANT_Y) {
            const float4 c4 = reinterpret_cast<const float4*>(bc + cofs)[q];
            Cv[4 * q] = c4.x; Cv[4 * q + 1] = c4.y; Cv[4 * q + 2] = c4.z; Cv[4 * q + 3] = c4.w;
        }
    }
    const float a = fast_exp2(dl * A2b);
    float p = r * (Q == 1 ? a : fast_exp2(dl * A2[0]));
    float y = 0.0f;
#pragma unroll
    for (int n = 0; n < SPL; ++n) {
        if (n) p *= a;
        g[n] = fmaf(p, g[n], Bv[n]);
        if (WANT_Y) y = n ? fmaf(Cv[n], g[n], y) : Cv[0] * g[0];
    }
    return y;
}

// Sum over the Q neighbouring lanes of a channel (Q = 1, 2, 4 or 8): quad_perm [1,0,3,2], then
// [2,3,0,1], then row_half_mirror (lane i of each eight takes lane 7 - i, the other quad); every
// lane of the group ends with the group's sum.
template <int Q>
__device__ __forceinline__ float group_sum(float v) {
    if (Q >= 2) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    if (Q >= 4) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    if (Q >= 8) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    return v;
}

// Per-wave tile geometry of the general kernels for storage E and d_state N.
template <class E, int N>
struct Geo {
    static constexpr int Q = Shape<N>::Q;
    static constexpr int CH = Shape<N>::CH;
    static constexpr int TT = Shape<N>::TT;
    static constexpr int V = E::kPerVec;          // elements per 16-byte vector
    static constexpr int CPR = TT / V;            // vectors per row per tile
    static constexpr int RPI = kRows / CPR;       // rows covered by one pass of the wave
    static constexpr int ITERS = (CH + RPI - 1) / RPI;  // passes to cover the CH rows
    static constexpr int BCHUNK = TT / 4;         // lanes per B / C row (four steps each)
    static constexpr int BROWS = kRows / BCHUNK;  // B / C rows per pass
    static constexpr int BPASS = (2 * N) / BROWS; // passes over the 2N rows of B | C
    static constexpr int BPW = BPASS / Shape<N>::WPB;  // of them, each wavefront's
    static_assert(TT % V == 0 && kRows % CPR == 0 && (CH % RPI == 0 || ITERS == 1), "tile shape");
    static_assert(BPASS % Shape<N>::WPB == 0, "B | C passes per wavefront");
};

// One tile's inputs in registers: u, delta, z in the coalesced layout and the B | C chunks.
template <class E, int N>
struct TileIn {
    uint4 u[Geo<E, N>::ITERS], d[Geo<E, N>::ITERS], z[Geo<E, N>::ITERS];
    float4 bc[Geo<E, N>::BPW];  // this wavefront's share of the B | C tile
};

// Issues every load of the tile starting at t0, at clamped addresses (row min(d, Dn - 1), step
// min(t, L - 1), or the last whole vector for vector rows) so that none needs a branch; values
// outside the tile's valid part are masked by the consumers.  (A load behind a branch would be
// waited for before the next one is issued.)
template <class E, bool VEC, bool WANT_Z, int N>
__device__ __forceinline__ void load_tile(const KArgs& a, TileIn<E, N>& in, const int lane, const int wave,
                                          const int b, const int64_t d0, const int64_t t0) {
    using G = Geo<E, N>;
    constexpr int V = G::V;
    const int64_t L = a.L, Dn = a.Dn;
#pragma unroll
    for (int it = 0; it < G::ITERS; ++it) {
        const int r = it * G::RPI + lane / G::CPR;
        const int tl = (lane % G::CPR) * V;
        const int64_t gd = d0 + r < Dn ? d0 + r : Dn - 1;
        const int64_t rowb = ((int64_t)b * Dn + gd) * L;
        if (VEC) {
            const int64_t tv = t0 + tl <= L - V ? t0 + tl : L - V;  // L is a multiple of V here
            in.u[it] = *reinterpret_cast<const uint4*>(static_cast<const typename E::storage*>(a.u) + rowb + tv);
            in.d[it] = *reinterpret_cast<const uint4*>(static_cast<const typename E::storage*>(a.delta) + rowb + tv);
            if (WANT_Z)
                in.z[it] = *reinterpret_cast<const uint4*>(static_cast<const typename E::storage*>(a.z) + rowb + tv);
        } else {
            float uv[V], dv[V], zv[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const int64_t te = t0 + tl + e < L ? t0 + tl + e : L - 1;
                uv[e] = E::load1(a.u, rowb + te);
                dv[e] = E::load1(a.delta, rowb + te);
                zv[e] = WANT_Z ? E::load1(a.z, rowb + te) : 0.0f;
            }
            in.u[it] = E::pack(uv);  // exact: values came from this storage type
            in.d[it] = E::pack(dv);
            in.z[it] = E::pack(zv);
        }
    }
    const int tlb = (lane % G::BCHUNK) * 4;
#pragma unroll
    for (int i = 0; i < G::BPW; ++i) {
        const int rr = (wave * G::BPW + i) * G::BROWS + lane / G::BCHUNK;
        const float* src = (rr < N ? a.B : a.C) + ((int64_t)b * N + (rr % N)) * L;
        if (VEC) {
            const int64_t tv = t0 + tlb <= L - 4 ? t0 + tlb : L - 4;  // L is a multiple of 4 here
            in.bc[i] = *reinterpret_cast<const float4*>(src + tv);
        } else {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = src[t0 + tlb + e < L ? t0 + tlb + e : L - 1];
            in.bc[i] = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
}

// Phase A of a tile: delta = softplus(raw + bias) and x = delta u into LDS in the coalesced
// layout, and B | C transposed to sm.bc[t][n]; padded steps and steps past the batch's length
// become identity updates (delta = 0, x = 0, B = C = 0, whatever the padding holds).
template <class E, int N>
__device__ __forceinline__ void stage_tile(const KArgs& a, Smem<N>& sm, const TileIn<E, N>& in, const int lane,
                                           const int wave, const int64_t d0, const int64_t t0, const int tvalid,
                                           const int64_t stop) {
    auto& w = sm.w[wave];
    using G = Geo<E, N>;
    constexpr int V = G::V;
#pragma unroll
    for (int it = 0; it < G::ITERS; ++it) {
        const int r = it * G::RPI + lane / G::CPR;
        if (G::CH % G::RPI != 0 && r >= G::CH) continue;  // lanes past the wave's rows (one pass only)
        const int tl = (lane % G::CPR) * V;
        const bool row_ok = d0 + r < a.Dn;
        float uv[V], dv[V];
        E::unpack(in.u[it], uv);
        E::unpack(in.d[it], dv);
        const float br = w.bias[r];
        float dl[V], xv[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float pre = dv[e] + br;
            float dlt = a.softplus ? softplus(pre) : pre;
            const bool live = row_ok && tl + e < tvalid && t0 + tl + e < stop;
            dl[e] = live ? dlt : 0.0f;
            xv[e] = live ? dlt * uv[e] : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < V / 4; ++q) {
            *reinterpret_cast<float4*>(&w.dl[r][tl + 4 * q]) =
                make_float4(dl[4 * q], dl[4 * q + 1], dl[4 * q + 2], dl[4 * q + 3]);
            *reinterpret_cast<float4*>(&w.x[r][tl + 4 * q]) =
                make_float4(xv[4 * q], xv[4 * q + 1], xv[4 * q + 2], xv[4 * q + 3]);
        }
    }
    const int tlb = (lane % G::BCHUNK) * 4;
#pragma unroll
    for (int i = 0; i < G::BPW; ++i) {
        const int rr = (wave * G::BPW + i) * G::BROWS + lane / G::BCHUNK;
        const float v[4] = {in.bc[i].x, in.bc[i].y, in.bc[i].z, in.bc[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            sm.bc[tlb + e][bc_word(rr)] = (tlb + e < tvalid && t0 + tlb + e < stop) ? v[e] : 0.0f;
    }
}

template <class E, bool VEC, bool HAS_Z, int MODE, bool POW, int N>
__device__ __forceinline__ void scan_body(const KArgs& a, Smem<N>& sm, const int lane, const int wave, const int b,
                                          const int64_t d0, const int64_t row, const bool active,
                                          const float (&A2)[Shape<N>::SPL], const float A2b,
                                          float (&h)[Shape<N>::SPL],
                                          const int64_t t_begin, const int64_t t_end, const int64_t stop) {
    using G = Geo<E, N>;
    constexpr int Q = G::Q;
    constexpr int CH = G::CH;
    constexpr int TT = G::TT;
    constexpr int V = G::V;
    constexpr bool WANT_Z = MODE == kMain && HAS_Z;
    constexpr int SPL = Shape<N>::SPL;

    const int64_t L = a.L;
    const int64_t Dn = a.Dn;
    const int cl = lane % G::CPR;        // vector column of this lane in the coalesced layout
    const int rl = lane / G::CPR;        // row offset of this lane within a pass
    const int c = lane / Q;              // this lane's channel within the wave (phase B)
    const int k = lane % Q;              // its block of SPL states
    auto& w = sm.w[wave];
    float dsum = 0.0f;
    constexpr bool SCALED = POW && SPL == 16;
    float sc = 1.0f;  // SCALED: h = sc * g, the array h holding g

    // (Issuing the next tile's loads before the recurrence, to hide their latency, measured no
    // faster at d_state 64 and 128: the other wavefronts on the SIMD already hide it.)
    for (int64_t t0 = t_begin; t0 < t_end; t0 += TT) {
        const int tvalid = static_cast<int>(t_end - t0 < TT ? t_end - t0 : TT);
        __syncthreads();  // the previous tile's readers of sm are done
        TileIn<E, N> in;
        load_tile<E, VEC, WANT_Z, N>(a, in, lane, wave, b, d0, t0);
        stage_tile<E, N>(a, sm, in, lane, wave, d0, t0, tvalid, stop);
        __syncthreads();

        // ---- phase B: the recurrence, lane = (channel, block of SPL states), sequential over the tile
        for (int tc = 0; tc < tvalid; tc += 4) {
            const float4 dl4 = *reinterpret_cast<const float4*>(&w.dl[c][tc]);
            const float4 x4 = *reinterpret_cast<const float4*>(&w.x[c][tc]);
            const float dlv[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
            const float xv[4] = {x4.x, x4.y, x4.z, x4.w};
            float yv[4], sv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (SCALED) {
                    sv[j] = step_scale(xv[j]);
                    yv[j] = step_lane_scaled<MODE == kMain, Q, SPL>(h, A2, A2b, dlv[j], sc * fast_rcp(sv[j]),
                                                                    &sm.bc[tc + j][bc_word(SPL * k)],
                                                                    bc_word(N + SPL * k) - bc_word(SPL * k));
                    sc = sv[j];
                } else {
                    yv[j] = step_lane<POW, MODE == kMain, Q, SPL>(h, A2, A2b, dlv[j], xv[j],
                                                                  &sm.bc[tc + j][bc_word(SPL * k)],
                                                                  bc_word(N + SPL * k) - bc_word(SPL * k));
                }
                if (MODE == kAgg) dsum += dlv[j];
            }
            if (MODE == kMain) {
#pragma unroll
                for (int j = 0; j < 4; ++j) yv[j] = SCALED ? sv[j] * group_sum<Q>(yv[j]) : group_sum<Q>(yv[j]);
                if (k == 0)
                    *reinterpret_cast<float4*>(&w.dl[c][tc]) = make_float4(yv[0], yv[1], yv[2], yv[3]);
            }
        }

        // ---- phase C: out = (y + D u) silu(z), coalesced stores
        if (MODE == kMain) {
            __syncthreads();
#pragma unroll
            for (int it = 0; it < G::ITERS; ++it) {
                const int r = it * G::RPI + rl;
                if (CH % G::RPI != 0 && r >= CH) continue;
                const int tl = cl * V;
                const int64_t gd = d0 + r;
                const int64_t base = ((int64_t)b * Dn + gd) * L + t0 + tl;
                const bool row_ok = gd < Dn;
                float uv[V], ov[V];
                E::unpack(in.u[it], uv);
                float zv[V];
                if (HAS_Z) E::unpack(in.z[it], zv);
                const float dr = w.dsk[r];
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float yy = fmaf(dr, uv[e], w.dl[r][tl + e]);
                    ov[e] = HAS_Z ? yy * silu(zv[e]) : yy;
                    if (t0 + tl + e >= stop) ov[e] = 0.0f;  // past the batch's length
                }
                if (VEC) {
                    if (row_ok && tl < tvalid)
                        *reinterpret_cast<uint4*>(static_cast<typename E::storage*>(a.out) + base) = E::pack(ov);
                } else {
#pragma unroll
                    for (int e = 0; e < V; ++e)
                        if (row_ok && tl + e < tvalid) E::store1(a.out, base + e, ov[e]);
                }
            }
        }
    }

    if (SCALED) {
#pragma unroll
        for (int n = 0; n < SPL; ++n) h[n] *= sc;  // back to the state itself
    }
    if (MODE == kMain) {
        if (a.last_state && active && blockIdx.z == a.S - 1) {
            float4* dst = reinterpret_cast<float4*>(a.last_state + row * N + SPL * k);
#pragma unroll
            for (int q = 0; q < SPL / 4; ++q)
                dst[q] = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
        }
    } else if (active) {
        float* ws = a.ws + (int64_t)blockIdx.z * (N + 1) * a.rows_total + row;
#pragma unroll
        for (int n = 0; n < SPL; ++n) ws[(int64_t)(SPL * k + n) * a.rows_total] = h[n];
        if (k == 0) ws[(int64_t)N * a.rows_total] = dsum;
    }
}

template <class E, bool VEC, bool HAS_Z, int MODE, int N>
__global__ __launch_bounds__(kRows * Shape<N>::WPB) __attribute__((amdgpu_waves_per_eu(N >= 32 ? 3 : 1))) void scan_kernel(KArgs a) {
    constexpr int Q = Shape<N>::Q;
    constexpr int CH = Shape<N>::CH;
    constexpr int SPL = Shape<N>::SPL;
    __shared__ Smem<N> sm;
    const int lane = threadIdx.x % kRows;
    const int wave = threadIdx.x / kRows;
    const int c = lane / Q, k = lane % Q;
    const int64_t d0 = ((int64_t)blockIdx.x * Shape<N>::WPB + wave) * CH;
    const int b = blockIdx.y;
    const int seg = blockIdx.z;
    const int64_t d = d0 + c;
    const bool active = d < a.Dn;
    const int64_t row = (int64_t)b * a.Dn + (active ? d : 0);

    float A2[SPL];
    float A2b = 0.0f;
    bool pow_ok = true;
    if (active) {
        const float4* Ar = reinterpret_cast<const float4*>(a.A + d * N + SPL * k);
        const float A0 = a.A[d * N];
        float Av[SPL];
#pragma unroll
        for (int q = 0; q < SPL / 4; ++q) {
            const float4 v = Ar[q];
            Av[4 * q] = v.x; Av[4 * q + 1] = v.y; Av[4 * q + 2] = v.z; Av[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int n = 0; n < SPL; ++n) {
            A2[n] = Av[n] * kLog2e;
            pow_ok = pow_ok && (Av[n] == static_cast<float>(SPL * k + n + 1) * A0);
        }
        A2b = A0 * kLog2e;
    } else {
#pragma unroll
        for (int n = 0; n < SPL; ++n) A2[n] = 0.0f;
    }
    if (k == 0) {
        sm.w[wave].bias[c] = (active && a.bias) ? a.bias[d] : 0.0f;
        sm.w[wave].dsk[c] = (active && a.D) ? a.D[d] : 0.0f;
    }

    float h[SPL];
    if (MODE == kMain && seg > 0 && active) {
        const float* ws = a.ws + (int64_t)(seg - 1) * (N + 1) * a.rows_total + row;
#pragma unroll
        for (int n = 0; n < SPL; ++n) h[n] = ws[(int64_t)(SPL * k + n) * a.rows_total];
    } else if (MODE == kMain && a.h0 && active) {
#pragma unroll
        for (int n = 0; n < SPL; ++n) h[n] = a.h0[row * N + SPL * k + n];
    } else {
#pragma unroll
        for (int n = 0; n < SPL; ++n) h[n] = 0.0f;
    }

    const int64_t t_begin = (int64_t)seg * a.seg_len;
    const int64_t t_end = (t_begin + a.seg_len < a.L) ? t_begin + a.seg_len : a.L;
    int64_t stop = a.L;
    if (a.lens) {
        const int64_t l = a.lens[b];
        stop = l < 0 ? 0 : (l > a.L ? a.L : l);
    }
    // (per wavefront; the wavefronts of a workgroup meet at the same barriers either way)
    if (__all(pow_ok))
        scan_body<E, VEC, HAS_Z, MODE, true, N>(a, sm, lane, wave, b, d0, row, active, A2, A2b, h, t_begin, t_end,
                                                stop);
    else
        scan_body<E, VEC, HAS_Z, MODE, false, N>(a, sm, lane, wave, b, d0, row, active, A2, A2b, h, t_begin, t_end,
                                                 stop);
}

// Folds the per-segment pairs (sum delta_s, local end state e_s) into inclusive end states:
// H_s = exp(A * sum delta_s) H_{s-1} + e_s, H_{-1} = h0 (zeros without one), written over e_s.
// One thread per (row, block of 16 states).
__global__ __launch_bounds__(256) void combine_kernel(KArgs a) {
    const int64_t R = a.rows_total;
    const int Q = a.N / 16;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < R * Q;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / Q;
        const int n0 = 16 * static_cast<int>(i % Q);
        const int64_t d = row % a.Dn;
        float A2[16], h[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            A2[n] = a.A[d * a.N + n0 + n] * kLog2e;
            h[n] = a.h0 ? a.h0[row * a.N + n0 + n] : 0.0f;
        }
        for (int s = 0; s + 1 < a.S; ++s) {
            float* ws = a.ws + (int64_t)s * (a.N + 1) * R + row;
            const float sd = ws[(int64_t)a.N * R];
#pragma unroll
            for (int n = 0; n < 16; ++n) {
                h[n] = fmaf(fast_exp2(sd * A2[n]), h[n], ws[(int64_t)(n0 + n) * R]);
                ws[(int64_t)(n0 + n) * R] = h[n];
            }
        }
    }
}

// L = 0: the final state is the starting state (h0, or zeros).
__global__ __launch_bounds__(256) void start_state_kernel(float* p, const float* h0, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = h0 ? h0[i] : 0.0f;
}

constexpr int kTile = 32;  // segment lengths are multiples of this (and of every Shape::TT)

template <class E, bool VEC, bool HAS_Z, int N>
hipError_t launch_typed(const KArgs& k, const ScanLaunch& a, hipStream_t stream) {
    const int64_t Bt = a.Bt;
    const dim3 block(kRows * Shape<N>::WPB);
    constexpr int CHB = Shape<N>::CH * Shape<N>::WPB;  // channels per workgroup
    const unsigned gx = static_cast<unsigned>((k.Dn + CHB - 1) / CHB);
    mark(a, 0, stream);
    if (k.S > 1) {
        scan_kernel<E, VEC, HAS_Z, kAgg, N><<<dim3(gx, (unsigned)Bt, (unsigned)(k.S - 1)), block, 0, stream>>>(k);
        const int64_t work = k.rows_total * (N / 16);
        const int64_t cblocks = (work + 255) / 256;
        combine_kernel<<<dim3((unsigned)(cblocks < 65535 ? cblocks : 65535)), dim3(256), 0, stream>>>(k);
    }
    mark(a, 1, stream);
    scan_kernel<E, VEC, HAS_Z, kMain, N><<<dim3(gx, (unsigned)Bt, (unsigned)k.S), block, 0, stream>>>(k);
    mark(a, 2, stream);
    return hipGetLastError();
}

template <class E, bool VEC, bool HAS_Z>
hipError_t launch_n(const KArgs& k, const ScanLaunch& a, hipStream_t stream) {
    switch (a.N) {
        case 16: return launch_typed<E, VEC, HAS_Z, 16>(k, a, stream);
        case 32: return launch_typed<E, VEC, HAS_Z, 32>(k, a, stream);
        case 64: return launch_typed<E, VEC, HAS_Z, 64>(k, a, stream);
        default: return launch_typed<E, VEC, HAS_Z, 128>(k, a, stream);
    }
}

}  // namespace

ScanPlan plan_scan(const ScanLaunch& a, int num_cus, int tile, int segments_override) {
    ScanPlan p;
    const int64_t spl = (a.N == 32 || a.N == 64) ? 8 : 16;   // states per lane (Shape<N>::SPL)
    const int64_t ch = kRows / (a.N / spl);   // channels per wavefront
    const int64_t wpb = a.N >= 32 ? 4 : 1;  // wavefronts per workgroup
    const int64_t groups = a.Bt * ((a.Dn + ch * wpb - 1) / (ch * wpb)) * wpb;
    const int64_t tiles = (a.L + tile - 1) / tile;
    // One wavefront per SIMD or more without a split: run unsplit (the aggregate pass a split adds
    // costs more than the fuller chip gains; at d_state 64, 4 x 5120 x 2048: 0.66 ms unsplit, 0.88
    // in two segments).  Fewer: split towards ~2 wavefronts per SIMD (4 SIMDs per CU), rounded.
    const int64_t simds = 4LL * (num_cus > 0 ? num_cus : 256);
    int64_t S = groups >= simds ? 1 : (2 * simds + groups / 2) / groups;
    if (segments_override > 0) S = segments_override;
    if (S < 1) S = 1;
    if (S > tiles) S = tiles > 0 ? tiles : 1;
    if (S > 65535) S = 65535;
    int64_t seg_tiles = (tiles + S - 1) / S;
    if (seg_tiles < 1) seg_tiles = 1;
    p.seg_len = seg_tiles * tile;
    p.segments = static_cast<int>(tiles > 0 ? (tiles + seg_tiles - 1) / seg_tiles : 1);
    p.waves = 0;
    p.xcds = 1;
    p.workspace_bytes = 0;
    return p;
}

int generic_tile() { return kTile; }

size_t generic_workspace_bytes(const ScanLaunch& a, int segments) {
    return segments > 1
        ? static_cast<size_t>(segments) * (a.N + 1) * static_cast<size_t>(a.Bt * a.Dn) * sizeof(float)
        : 0;
}

hipError_t launch_scan_fwd(const ScanLaunch& a, const ScanPlan& plan, float* workspace,
                           hipStream_t stream) {
    const int64_t rows = a.Bt * a.Dn;
    if (rows == 0) return hipSuccess;
    if (a.L == 0) {
        if (a.last_state) {
            const int64_t n = rows * a.N;
            const int64_t blocks = (n + 255) / 256;
            start_state_kernel<<<dim3((unsigned)(blocks < 65535 ? blocks : 65535)), dim3(256), 0, stream>>>(
                a.last_state, a.h0, n);
            return hipGetLastError();
        }
        return hipSuccess;
    }
    KArgs k;
    k.u = a.u; k.delta = a.delta; k.z = a.z; k.A = a.A; k.B = a.B; k.C = a.C; k.D = a.D;
    k.bias = a.bias; k.out = a.out; k.last_state = a.last_state; k.h0 = a.h0; k.lens = a.lens; k.ws = workspace;
    k.Dn = a.Dn; k.L = a.L; k.seg_len = plan.seg_len; k.rows_total = rows;
    k.S = plan.segments; k.N = a.N; k.softplus = a.softplus;
    const bool hz = a.z != nullptr;
    if (a.bf16) {
        if (a.vec_ok) return hz ? launch_n<BF16, true, true>(k, a, stream) : launch_n<BF16, true, false>(k, a, stream);
        return hz ? launch_n<BF16, false, true>(k, a, stream) : launch_n<BF16, false, false>(k, a, stream);
    }
    if (a.vec_ok) return hz ? launch_n<F32, true, true>(k, a, stream) : launch_n<F32, true, false>(k, a, stream);
    return hz ? launch_n<F32, false, true>(k, a, stream) : launch_n<F32, false, false>(k, a, stream);
}

}  // namespace mss
