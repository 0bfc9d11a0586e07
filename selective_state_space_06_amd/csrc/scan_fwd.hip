// scan_fwd.hip -- forward selective scan (S6) for gfx950.
//
// Computes, per batch b, channel d and state n (Mamba paper Section 3 / Algorithm 2, as
// coded on the Keras/TensorFlow Mamba tutorial page in `selective_scan` and
// `MambaBlock.ssm`; the upstream mamba README's "Selective SSM" layer):
//   delta_t = softplus(delta_raw_t + bias_d)   Abar = exp(delta_t A_dn)
//   h_t = Abar h_{t-1} + delta_t B_nt u_t (h_0 = 0, or a given state)
//   out_t = (sum_n C_nt h_t + D_d u_t) silu(z_t)
//
// Work decomposition (one wavefront per workgroup):
//   * a lane owns one channel (row b, d) and keeps its 16 states in VGPRs, sequential in t;
//   * the 64 lanes of a wave are 64 consecutive channels of one batch, so B_t and C_t are
//     the same for every lane: they are staged once per time tile in LDS, transposed to
//     [t][n], and read back as broadcast 16-byte LDS loads;
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
// tutorial uses), Abar_n = Abar_0^(n+1) is formed by repeated multiplication: one exp2 per
// (b, d, t) instead of sixteen.  The choice is made per wavefront on the device from the A
// rows it loads; any other A takes the general path.
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
    const float* h0;      // nullable starting state, (rows_total, kN)
    const int32_t* lens;  // nullable per-batch sequence lengths
    float* ws;            // [S][kN + 1][rows_total] carry workspace
    int64_t Dn, L, seg_len, rows_total;
    int S;
    int softplus;
};

template <int TT>
struct Smem {
    static constexpr int kRowStride = TT + 4;   // 16-byte pad: lane-row 16 B reads hit distinct banks
    static constexpr int kBCStride = 2 * kN + 4;
    float dl[kRows][kRowStride];  // delta (phase A) then y (phase B)
    float x[kRows][kRowStride];   // delta * u
    float bc[TT][kBCStride];      // B[0..15] | C[0..15] per time step
    float bias[kRows];
    float dsk[kRows];
};

// One time step of one lane: 16 state updates and (main pass) the C.h reduction.
template <bool POW, bool WANT_Y>
__device__ __forceinline__ float step16(float (&h)[kN], const float (&A2)[kN], float dl, float x,
                                        const float* __restrict__ bc) {
    float Bv[kN], Cv[kN];
#pragma unroll
    for (int q = 0; q < kN / 4; ++q) {
        const float4 b4 = reinterpret_cast<const float4*>(bc)[q];
        Bv[4 * q] = b4.x; Bv[4 * q + 1] = b4.y; Bv[4 * q + 2] = b4.z; Bv[4 * q + 3] = b4.w;
        if (WANT_Y) {
            const float4 c4 = reinterpret_cast<const float4*>(bc + kN)[q];
            Cv[4 * q] = c4.x; Cv[4 * q + 1] = c4.y; Cv[4 * q + 2] = c4.z; Cv[4 * q + 3] = c4.w;
        }
    }
    float y = 0.0f;
    if (POW) {
        const float a = fast_exp2(dl * A2[0]);
        float p = a;
#pragma unroll
        for (int n = 0; n < kN; ++n) {
            if (n) p *= a;
            h[n] = fmaf(p, h[n], x * Bv[n]);
            if (WANT_Y) y = n ? fmaf(Cv[n], h[n], y) : Cv[0] * h[0];
        }
    } else {
#pragma unroll
        for (int n = 0; n < kN; ++n) {
            h[n] = fmaf(fast_exp2(dl * A2[n]), h[n], x * Bv[n]);
            if (WANT_Y) y = n ? fmaf(Cv[n], h[n], y) : Cv[0] * h[0];
        }
    }
    return y;
}

template <class E, bool VEC, bool HAS_Z, int MODE, bool POW, int TT>
__device__ __forceinline__ void scan_body(const KArgs& a, Smem<TT>& sm, const int lane, const int b,
                                          const int64_t d0, const int64_t row, const bool active,
                                          const float (&A2)[kN], float (&h)[kN],
                                          const int64_t t_begin, const int64_t t_end, const int64_t stop) {
    constexpr int V = E::kPerVec;        // elements per 16-byte vector
    constexpr int CPR = TT / V;          // vectors per row per tile
    constexpr int RPI = kRows / CPR;     // rows covered by one pass of the wave
    constexpr int ITERS = CPR;           // passes to cover the 64 rows
    static_assert(TT % V == 0 && kRows % CPR == 0, "tile shape");

    const int64_t L = a.L;
    const int64_t Dn = a.Dn;
    const int cl = lane % CPR;           // vector column of this lane in the coalesced layout
    const int rl = lane / CPR;           // row offset of this lane within a pass
    float dsum = 0.0f;

    for (int64_t t0 = t_begin; t0 < t_end; t0 += TT) {
        const int tvalid = static_cast<int>(t_end - t0 < TT ? t_end - t0 : TT);
        __syncthreads();  // the previous tile's readers of sm are done

        // ---- phase A: coalesced loads of u / delta, delta = softplus(raw + bias), x = delta u
        uint4 uraw[ITERS];
        uint4 zraw[ITERS];
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            const int r = it * RPI + rl;
            const int tl = cl * V;
            const int64_t gd = d0 + r;
            const int64_t base = ((int64_t)b * Dn + gd) * L + t0 + tl;
            const bool row_ok = gd < Dn;
            float uv[V], dv[V];
            if (VEC) {
                uint4 wu = make_uint4(0, 0, 0, 0), wd = make_uint4(0, 0, 0, 0);
                if (row_ok && tl < tvalid) {
                    wu = *reinterpret_cast<const uint4*>(static_cast<const typename E::storage*>(a.u) + base);
                    wd = *reinterpret_cast<const uint4*>(static_cast<const typename E::storage*>(a.delta) + base);
                }
                uraw[it] = wu;
                E::unpack(wu, uv);
                E::unpack(wd, dv);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const bool ok = row_ok && tl + e < tvalid;
                    uv[e] = ok ? E::load1(a.u, base + e) : 0.0f;
                    dv[e] = ok ? E::load1(a.delta, base + e) : 0.0f;
                }
                uraw[it] = E::pack(uv);  // exact: values came from this storage type
            }
            const float br = sm.bias[r];
            float dl[V], xv[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float pre = dv[e] + br;
                float dlt = a.softplus ? softplus(pre) : pre;
                // padded steps and steps past the batch's length: identity update
                const bool live = row_ok && tl + e < tvalid && t0 + tl + e < stop;
                dl[e] = live ? dlt : 0.0f;
                xv[e] = live ? dlt * uv[e] : 0.0f;
            }
#pragma unroll
            for (int q = 0; q < V / 4; ++q) {
                *reinterpret_cast<float4*>(&sm.dl[r][tl + 4 * q]) =
                    make_float4(dl[4 * q], dl[4 * q + 1], dl[4 * q + 2], dl[4 * q + 3]);
                *reinterpret_cast<float4*>(&sm.x[r][tl + 4 * q]) =
                    make_float4(xv[4 * q], xv[4 * q + 1], xv[4 * q + 2], xv[4 * q + 3]);
            }
        }
        // B / C tile -> sm.bc[t][n] (transposed); 32 rows (16 of B, 16 of C) x TT steps
        {
            constexpr int BCHUNK = TT / 4;              // 4-float chunks per row
            constexpr int BROWS = kRows / BCHUNK;       // rows per pass
#pragma unroll
            for (int it = 0; it < (2 * kN) / BROWS; ++it) {
                const int rr = it * BROWS + lane / BCHUNK;
                const int tl = (lane % BCHUNK) * 4;
                const float* src = (rr < kN ? a.B : a.C) + ((int64_t)b * kN + (rr % kN)) * L + t0 + tl;
#pragma unroll
                for (int e = 0; e < 4; ++e)  // past the batch's length: zeros, whatever the padding holds
                    sm.bc[tl + e][rr] = (tl + e < tvalid && t0 + tl + e < stop) ? src[e] : 0.0f;
            }
        }
        // prefetch z for phase C while the recurrence runs
        if (MODE == kMain && HAS_Z) {
#pragma unroll
            for (int it = 0; it < ITERS; ++it) {
                const int r = it * RPI + rl;
                const int tl = cl * V;
                const int64_t gd = d0 + r;
                const int64_t base = ((int64_t)b * Dn + gd) * L + t0 + tl;
                const bool row_ok = gd < Dn;
                if (VEC) {
                    zraw[it] = (row_ok && tl < tvalid)
                        ? *reinterpret_cast<const uint4*>(static_cast<const typename E::storage*>(a.z) + base)
                        : make_uint4(0, 0, 0, 0);
                } else {
                    float zv[V];
#pragma unroll
                    for (int e = 0; e < V; ++e)
                        zv[e] = (row_ok && tl + e < tvalid) ? E::load1(a.z, base + e) : 0.0f;
                    zraw[it] = E::pack(zv);
                }
            }
        }
        __syncthreads();

        // ---- phase B: the recurrence, lane = channel, sequential over the tile
        for (int tc = 0; tc < tvalid; tc += 4) {
            const float4 dl4 = *reinterpret_cast<const float4*>(&sm.dl[lane][tc]);
            const float4 x4 = *reinterpret_cast<const float4*>(&sm.x[lane][tc]);
            const float dlv[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
            const float xv[4] = {x4.x, x4.y, x4.z, x4.w};
            float yv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                yv[j] = step16<POW, MODE == kMain>(h, A2, dlv[j], xv[j], &sm.bc[tc + j][0]);
                if (MODE == kAgg) dsum += dlv[j];
            }
            if (MODE == kMain)
                *reinterpret_cast<float4*>(&sm.dl[lane][tc]) = make_float4(yv[0], yv[1], yv[2], yv[3]);
        }

        // ---- phase C: out = (y + D u) silu(z), coalesced stores
        if (MODE == kMain) {
            __syncthreads();
#pragma unroll
            for (int it = 0; it < ITERS; ++it) {
                const int r = it * RPI + rl;
                const int tl = cl * V;
                const int64_t gd = d0 + r;
                const int64_t base = ((int64_t)b * Dn + gd) * L + t0 + tl;
                const bool row_ok = gd < Dn;
                float uv[V], ov[V];
                E::unpack(uraw[it], uv);
                float zv[V];
                if (HAS_Z) E::unpack(zraw[it], zv);
                const float dr = sm.dsk[r];
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float yy = fmaf(dr, uv[e], sm.dl[r][tl + e]);
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

    if (MODE == kMain) {
        if (a.last_state && active && blockIdx.z == a.S - 1) {
            float4* dst = reinterpret_cast<float4*>(a.last_state + row * kN);
#pragma unroll
            for (int q = 0; q < kN / 4; ++q)
                dst[q] = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
        }
    } else if (active) {
        float* ws = a.ws + (int64_t)blockIdx.z * (kN + 1) * a.rows_total + row;
#pragma unroll
        for (int n = 0; n < kN; ++n) ws[(int64_t)n * a.rows_total] = h[n];
        ws[(int64_t)kN * a.rows_total] = dsum;
    }
}

template <class E, bool VEC, bool HAS_Z, int MODE, int TT>
__global__ __launch_bounds__(kRows) void scan_kernel(KArgs a) {
    __shared__ Smem<TT> sm;
    const int lane = threadIdx.x;
    const int64_t d0 = (int64_t)blockIdx.x * kRows;
    const int b = blockIdx.y;
    const int seg = blockIdx.z;
    const int64_t d = d0 + lane;
    const bool active = d < a.Dn;
    const int64_t row = (int64_t)b * a.Dn + (active ? d : 0);

    float A2[kN];
    bool pow_ok = true;
    if (active) {
        const float4* Ar = reinterpret_cast<const float4*>(a.A + d * kN);
        float Av[kN];
#pragma unroll
        for (int q = 0; q < kN / 4; ++q) {
            const float4 v = Ar[q];
            Av[4 * q] = v.x; Av[4 * q + 1] = v.y; Av[4 * q + 2] = v.z; Av[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int n = 0; n < kN; ++n) {
            A2[n] = Av[n] * kLog2e;
            pow_ok = pow_ok && (Av[n] == static_cast<float>(n + 1) * Av[0]);
        }
    } else {
#pragma unroll
        for (int n = 0; n < kN; ++n) A2[n] = 0.0f;
    }
    sm.bias[lane] = (active && a.bias) ? a.bias[d] : 0.0f;
    sm.dsk[lane] = (active && a.D) ? a.D[d] : 0.0f;

    float h[kN];
    if (MODE == kMain && seg > 0 && active) {
        const float* ws = a.ws + (int64_t)(seg - 1) * (kN + 1) * a.rows_total + row;
#pragma unroll
        for (int n = 0; n < kN; ++n) h[n] = ws[(int64_t)n * a.rows_total];
    } else if (MODE == kMain && a.h0 && active) {
#pragma unroll
        for (int n = 0; n < kN; ++n) h[n] = a.h0[row * kN + n];
    } else {
#pragma unroll
        for (int n = 0; n < kN; ++n) h[n] = 0.0f;
    }

    const int64_t t_begin = (int64_t)seg * a.seg_len;
    const int64_t t_end = (t_begin + a.seg_len < a.L) ? t_begin + a.seg_len : a.L;
    int64_t stop = a.L;
    if (a.lens) {
        const int64_t l = a.lens[b];
        stop = l < 0 ? 0 : (l > a.L ? a.L : l);
    }
    if (__all(pow_ok))
        scan_body<E, VEC, HAS_Z, MODE, true, TT>(a, sm, lane, b, d0, row, active, A2, h, t_begin, t_end, stop);
    else
        scan_body<E, VEC, HAS_Z, MODE, false, TT>(a, sm, lane, b, d0, row, active, A2, h, t_begin, t_end, stop);
}

// Folds the per-segment pairs (sum delta_s, local end state e_s) into inclusive end states:
// H_s = exp(A * sum delta_s) H_{s-1} + e_s, H_{-1} = h0 (zeros without one), written over e_s.
__global__ __launch_bounds__(256) void combine_kernel(KArgs a) {
    const int64_t R = a.rows_total;
    for (int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; row < R;
         row += (int64_t)gridDim.x * blockDim.x) {
        const int64_t d = row % a.Dn;
        float A2[kN], h[kN];
#pragma unroll
        for (int n = 0; n < kN; ++n) {
            A2[n] = a.A[d * kN + n] * kLog2e;
            h[n] = a.h0 ? a.h0[row * kN + n] : 0.0f;
        }
        for (int s = 0; s + 1 < a.S; ++s) {
            float* ws = a.ws + (int64_t)s * (kN + 1) * R + row;
            const float sd = ws[(int64_t)kN * R];
#pragma unroll
            for (int n = 0; n < kN; ++n) {
                h[n] = fmaf(fast_exp2(sd * A2[n]), h[n], ws[(int64_t)n * R]);
                ws[(int64_t)n * R] = h[n];
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

constexpr int kTile = 32;

template <class E, bool VEC, bool HAS_Z>
hipError_t launch_typed(const KArgs& k, const ScanLaunch& a, hipStream_t stream) {
    const int64_t Bt = a.Bt;
    const dim3 block(kRows);
    const unsigned gx = static_cast<unsigned>((k.Dn + kRows - 1) / kRows);
    mark(a, 0, stream);
    if (k.S > 1) {
        scan_kernel<E, VEC, HAS_Z, kAgg, kTile><<<dim3(gx, (unsigned)Bt, (unsigned)(k.S - 1)), block, 0, stream>>>(k);
        const int64_t cblocks = (k.rows_total + 255) / 256;
        combine_kernel<<<dim3((unsigned)(cblocks < 65535 ? cblocks : 65535)), dim3(256), 0, stream>>>(k);
    }
    mark(a, 1, stream);
    scan_kernel<E, VEC, HAS_Z, kMain, kTile><<<dim3(gx, (unsigned)Bt, (unsigned)k.S), block, 0, stream>>>(k);
    mark(a, 2, stream);
    return hipGetLastError();
}

}  // namespace

ScanPlan plan_scan(const ScanLaunch& a, int num_cus, int tile, int segments_override) {
    ScanPlan p;
    const int64_t groups = a.Bt * ((a.Dn + kRows - 1) / kRows);
    const int64_t tiles = (a.L + tile - 1) / tile;
    // aim for ~2 wavefronts per SIMD (4 SIMDs per CU) across the whole launch
    const int64_t target = 8LL * (num_cus > 0 ? num_cus : 256);
    int64_t S = (target + groups - 1) / groups;
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
        ? static_cast<size_t>(segments) * (kN + 1) * static_cast<size_t>(a.Bt * a.Dn) * sizeof(float)
        : 0;
}

hipError_t launch_scan_fwd(const ScanLaunch& a, const ScanPlan& plan, float* workspace,
                           hipStream_t stream) {
    const int64_t rows = a.Bt * a.Dn;
    if (rows == 0) return hipSuccess;
    if (a.L == 0) {
        if (a.last_state) {
            const int64_t n = rows * kN;
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
    k.S = plan.segments; k.softplus = a.softplus;
    const bool hz = a.z != nullptr;
    if (a.bf16) {
        if (a.vec_ok) return hz ? launch_typed<BF16, true, true>(k, a, stream) : launch_typed<BF16, true, false>(k, a, stream);
        return hz ? launch_typed<BF16, false, true>(k, a, stream) : launch_typed<BF16, false, false>(k, a, stream);
    }
    if (a.vec_ok) return hz ? launch_typed<F32, true, true>(k, a, stream) : launch_typed<F32, true, false>(k, a, stream);
    return hz ? launch_typed<F32, false, true>(k, a, stream) : launch_typed<F32, false, false>(k, a, stream);
}

}  // namespace mss
