// scan_bwd.hip -- gradients of the forward selective scan (S6) for gfx950.
//
// The forward (Keras/TensorFlow Mamba tutorial page, `selective_scan` and `MambaBlock.ssm` /
// `MambaBlock.call`; Mamba paper Section 3 as that page restates it):
//   pre = delta_raw + bias, dt = softplus(pre) (or pre), abar_n = exp(dt A_n),
//   h_t = abar_t h_{t-1} + dt_t B_t u_t (h_0 = 0), y_t = C_t.h_t + D u_t, out_t = y_t silu(z_t).
// The pages give no backward; this is the forward's reverse-mode derivative by the chain
// rule.  With dy_t = dout_t silu(z_t) and G_t = dL/dh_t = dy_t C_t + abar_{t+1} G_{t+1}:
//   du_t     = dt_t sum_n G_tn B_tn + D dy_t
//   ddelta_t = sigmoid(pre_t) sum_n G_tn (A_n abar_tn h_{t-1,n} + B_tn u_t)   (softplus on)
//   dz_t     = dout_t y_t silu'(z_t),  silu'(z) = s (1 + z (1 - s)), s = sigmoid(z)
//   dA_dn    = sum_{b,t} G_tn dt_t abar_tn h_{t-1,n},  dD_d = sum dy u,  dbias_d = sum ddelta
//   dB_bnt   = sum_d G_tn dt_t u_t,  dC_bnt = sum_d dy_t h_tn
// abar h_{t-1} is taken as h_t - dt B u (no second copy of the state), exp as exp2 of a
// log2(e)-prescaled argument, and A = (n + 1) A_0 rows use abar_n = abar_0^(n+1) as in the
// forward.  The forward may start from a given h0 and stop at a per-batch length (as the forward
// entry points allow); a gradient of the final state, dL/dh_L, seeds the adjoint at the last
// step, and dL/dh0 is the adjoint left after step 0.
//
// Decomposition (one wavefront per workgroup; lane = channel, 16 states in VGPRs):
//   * each channel row is cut into S segments of whole 8-step tiles.  An aggregate kernel walks
//     every segment forward from h = 0 and writes, per tile, a checkpoint (the tile's start
//     state from h = 0 at the segment start, and the sum of dt so far), and per segment its
//     forward carry (sum of dt, end state) and its adjoint carry
//     Lambda = sum_t (prod of abar over the segment's steps up to t) dy_t C_t, the part of
//     dL/dh that flows out of the segment's first step into the one before;
//   * the main kernel folds the forward carries of the earlier segments into the state h_in
//     entering its segment and the adjoint carries of the later segments (the same associative
//     operator, taken in reverse order) into the adjoint entering its last step, then walks its
//     tiles backward.  A tile's true start state is exp(A sum dt) h_in + its checkpoint (the
//     recurrence is linear); its states are recomputed from there into LDS, 8 at a time, and
//     consumed in reverse;
//   * dB and dC sum over channels: per step the wave's 64 x 32 terms are summed over its lanes
//     with cross-lane swaps and DPP (no LDS); a reduction kernel adds the per-wave sums of the
//     channel groups.
//     dA / dD / dbias are per-lane sums, added over segments and batches by a second kernel.
// Every sum is taken in a fixed order, so results do not vary from run to run.
#include <cstdlib>

#include "device_math.hpp"
#include "mss_internal.hpp"

namespace mss {
namespace {

constexpr int kBT = 8;            // steps per tile
constexpr int kAggW = 2 * kN + 1; // aggregate words per (segment, row): sum dt | H[16] | Lambda[16]
constexpr int kParW = kN + 2;     // partial words per (segment, row): dA[16] | dD | dbias
constexpr int kBCs = 2 * kN + 4;  // LDS words per step of B | C (16-byte pad)
constexpr int kCkW = kN + 1;      // checkpoint words per (tile, row): local state[16] | sum dt
// Steps whose recomputed states the main kernel keeps in LDS at once: four for bf16 rows (13 KB
// of LDS in all: eight wavefronts per CU, as many as the registers allow), the whole tile for
// fp32 rows (21 KB: seven per CU; their larger prefetched tiles leave no registers for the
// re-walk a smaller buffer costs, which measured slower).
template <class E>
constexpr int q_steps() { return sizeof(typename E::storage) == 2 ? 4 : kBT; }

struct BwdArgs {
    const void* u;
    const void* delta;
    const void* z;
    const void* dout;
    const float* A;
    const float* B;
    const float* C;
    const float* D;
    const float* bias;
    void* du;
    void* ddelta;
    void* dz;
    const float* h0;     // nullable starting state (R, kN)
    const int32_t* lens; // nullable per-batch lengths
    const float* dlast;  // nullable dL/d last_state (R, kN)
    float* dh0;          // nullable dL/dh0 (R, kN), written by segment 0
    const float* saved;  // nullable: the forward's state entering each tile, [ntiles][kN / 4][R][4]
    float* agg;   // [S][kAggW][R]
    float* ck;    // [ntiles][kCkW][R]
    float* part;  // [G][Bt][2 kN][tpad]
    float* par;   // [S][kParW][R]
    int64_t Dn, L, R, ntiles, tpad;
    int S, G, Bt;
};

struct Row {
    int64_t row;      // flat (b, d) row, clamped to a valid row for inactive lanes
    bool active;
    float A2[kN];     // A * log2(e)
    float An[kN];     // A
    float bias, dskip;
    bool pow_ok;
    int64_t stop;     // the batch's sequence length: later steps take no part
};

__device__ __forceinline__ Row row_of(const BwdArgs& a) {
    Row r;
    const int64_t d = (int64_t)blockIdx.x * 64 + threadIdx.x;
    r.active = d < a.Dn;
    const int64_t dc = r.active ? d : a.Dn - 1;
    r.row = (int64_t)blockIdx.y * a.Dn + dc;
    const float4* Ar = reinterpret_cast<const float4*>(a.A + dc * kN);
#pragma unroll
    for (int q = 0; q < kN / 4; ++q) {
        const float4 v = Ar[q];
        r.An[4 * q] = v.x; r.An[4 * q + 1] = v.y; r.An[4 * q + 2] = v.z; r.An[4 * q + 3] = v.w;
    }
    r.pow_ok = true;
#pragma unroll
    for (int n = 0; n < kN; ++n) {
        r.A2[n] = r.An[n] * kLog2e;
        r.pow_ok = r.pow_ok && (r.An[n] == static_cast<float>(n + 1) * r.An[0]);
    }
    r.bias = a.bias ? a.bias[dc] : 0.0f;
    if (a.lens) {
        const int64_t l = a.lens[blockIdx.y];
        r.stop = l < 0 ? 0 : (l > a.L ? a.L : l);
    } else {
        r.stop = a.L;
    }
    r.dskip = a.D ? a.D[dc] : 0.0f;
    return r;
}

// abar_n for one step: exp2(dt A2_n), or abar_0^(n+1) by a product tree on the power path.
template <bool POW>
__device__ __forceinline__ void abar16(float dt, const float (&A2)[kN], float (&p)[kN]) {
    if (POW) {
        const float a = fast_exp2(dt * A2[0]);
        p[0] = a;
        p[1] = a * a;
        p[2] = p[1] * a;
        p[3] = p[1] * p[1];
#pragma unroll
        for (int k = 0; k < 4; ++k) p[4 + k] = p[3] * p[k];
#pragma unroll
        for (int k = 0; k < 8; ++k) p[8 + k] = p[7] * p[k];
    } else {
#pragma unroll
        for (int n = 0; n < kN; ++n) p[n] = fast_exp2(dt * A2[n]);
    }
}

constexpr int kH = kN / 2;  // states per half-pass of the backward walk

// exp2(dt A2_n) for the 8 states kH * hf .. kH * hf + 7; on the power path from a0 = exp2(dt A2_0)
// by multiplications.
template <bool POW>
__device__ __forceinline__ void abar8(float dt, float a0, const float (&A2)[kN], int hf, float (&p)[kH]) {
    if (POW) {
        const float a = a0;
        p[0] = a;
        p[1] = a * a;
        p[2] = p[1] * a;
        p[3] = p[1] * p[1];
#pragma unroll
        for (int k = 0; k < 4; ++k) p[4 + k] = p[3] * p[k];
        if (hf) {
            const float a8 = p[7];
#pragma unroll
            for (int k = 0; k < kH; ++k) p[k] *= a8;
        }
    } else {
#pragma unroll
        for (int k = 0; k < kH; ++k) p[k] = fast_exp2(dt * A2[kH * hf + k]);
    }
}

// Sums 16 per-lane terms over the 64 lanes without LDS, halving the number of values per lane
// at each level: across the wave halves (permlane32 swap), across row pairs (permlane16 swap),
// then within 16-lane rows by DPP (lane + 8 of the row, the mirrored lane of each half-row,
// lane ^ 2, lane ^ 1).  Every lane ends with the full sum of term sum16_term(lane); the four
// lanes of a quad hold the same term.  gfx950's swaps exchange rows between two registers:
// permlane16_swap(a, b) returns rows (a0, b0, a2, b2) and (a1, b1, a3, b3) of the 16-lane rows,
// permlane32_swap(a, b) the halves (a_lo, b_lo) and (a_hi, b_hi); the sum of the pair is then
// b's term summed over the row pair (or halves) in the odd rows (upper half), a's in the others.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ int sum16_term(int lane) {
    const int b2 = (lane >> 2) & 1, b3 = (lane >> 3) & 1, odd = (lane >> 4) & 1, hi = (lane >> 5) & 1;
    return b2 + 2 * b3 + 4 * (1 - odd) + 8 * (1 - hi);
}

__device__ __forceinline__ float lanes_sum16(const float (&t)[16]) {
    const int lane = threadIdx.x & 63;
    float u[8], v[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // lanes 0..31 keep term i + 8, lanes 32..63 term i
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(t[i + 8]), __float_as_uint(t[i]), false, false);
        u[i] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // even rows keep u[i + 4], odd rows u[i]
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(u[i + 4]), __float_as_uint(u[i]), false, false);
        v[i] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    }
    const bool b3 = (lane >> 3) & 1, b2 = (lane >> 2) & 1;
    // with lane + 8 of the row: bit 3 clear keeps v[0], v[1], set keeps v[2], v[3]
    const float w0 = (b3 ? v[2] : v[0]) + dpp_f<0x128>(b3 ? v[0] : v[2]);
    const float w1 = (b3 ? v[3] : v[1]) + dpp_f<0x128>(b3 ? v[1] : v[3]);
    // with the mirrored lane of the half-row (bit 2 differs): bit 2 clear keeps w0, set keeps w1
    float x = (b2 ? w1 : w0) + dpp_f<0x141>(b2 ? w0 : w1);
    x += dpp_f<0x4E>(x);  // lane ^ 2
    x += dpp_f<0xB1>(x);  // lane ^ 1
    return x;
}

__device__ __forceinline__ float sigmoid(float v) { return fast_rcp(1.0f + fast_exp2(-v * kLog2e)); }

// One tile (kBT steps from t0) of the lane's row into the output.  VEC: whole aligned 16-byte
// vectors (L is then a multiple of the vector length, so a vector is entirely valid or entirely
// past the end).  Otherwise (rows of any length, element-aligned): element-aligned 16-byte
// stores, and the vector that crosses the row's end element by element.
template <class E, bool VEC>
__device__ __forceinline__ void store_tile(void* base, int64_t off, int64_t t0, int64_t L,
                                           const float (&v)[kBT]) {
    typename E::storage* p = static_cast<typename E::storage*>(base) + off;
    constexpr int V = E::kPerVec;
#pragma unroll
    for (int q = 0; q < kBT / V; ++q) {
        const int64_t t = t0 + q * V;
        if (VEC) {
            if (t < L) *reinterpret_cast<uint4*>(p + t) = E::pack(&v[q * V]);
        } else if (t + V <= L) {
            const uint4 w = E::pack(&v[q * V]);
            __builtin_memcpy(p + t, &w, 16);
        } else {
#pragma unroll
            for (int e = 0; e < V; ++e)
                if (t + e < L) E::store1(p, t + e, v[q * V + e]);
        }
    }
}

__device__ __forceinline__ void read_bc(const float* sbc, int j, float (&bv)[kN], float (&cv)[kN]) {
    const float4* b4 = reinterpret_cast<const float4*>(sbc + j * kBCs);
#pragma unroll
    for (int q = 0; q < kN / 4; ++q) {
        const float4 x = b4[q], y = b4[kN / 4 + q];
        bv[4 * q] = x.x; bv[4 * q + 1] = x.y; bv[4 * q + 2] = x.z; bv[4 * q + 3] = x.w;
        cv[4 * q] = y.x; cv[4 * q + 1] = y.y; cv[4 * q + 2] = y.z; cv[4 * q + 3] = y.w;
    }
}

// B and C of the 8 states of half hf at tile step j.
__device__ __forceinline__ void read_bc_half(const float* sbc, int j, int hf, float (&bv)[kH], float (&cv)[kH]) {
    const float4* b4 = reinterpret_cast<const float4*>(sbc + j * kBCs + kH * hf);
    const float4* c4 = reinterpret_cast<const float4*>(sbc + j * kBCs + kN + kH * hf);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const float4 x = b4[q], y = c4[q];
        bv[4 * q] = x.x; bv[4 * q + 1] = x.y; bv[4 * q + 2] = x.z; bv[4 * q + 3] = x.w;
        cv[4 * q] = y.x; cv[4 * q + 1] = y.y; cv[4 * q + 2] = y.z; cv[4 * q + 3] = y.w;
    }
}

// One tile of the lane's inputs as loaded (the 16-byte vectors, converted when used, so the
// loads of the next tile can be in flight while this one is computed), plus the lane's four
// B or C values for the tile's LDS block.
template <class E, bool VEC>
struct Raw {
    static constexpr int NV = kBT * static_cast<int>(sizeof(typename E::storage)) / 16;
    uint4 u[NV], d[NV], g[NV], z[NV];
    float bc[4];
};

// The tile's vectors of one array; past the row's end they read as zeros.  VEC: aligned 16-byte
// loads.  Otherwise (rows of any length): element-aligned 16-byte loads, and the vector that
// crosses the row's end element by element, so no load leaves the row's tensor.  (t0 and L are
// the same for every lane: the choice is uniform.)
template <class E, bool VEC>
__device__ __forceinline__ void raw_row(const void* base, int64_t off, int64_t t0, int64_t L,
                                        uint4 (&w)[Raw<E, true>::NV]) {
    const typename E::storage* p = static_cast<const typename E::storage*>(base) + off;
    constexpr int V = E::kPerVec;
#pragma unroll
    for (int q = 0; q < Raw<E, true>::NV; ++q) {
        const int64_t t = t0 + q * V;
        if (VEC) {
            w[q] = t < L ? *reinterpret_cast<const uint4*>(p + t) : make_uint4(0, 0, 0, 0);
        } else if (t + V <= L) {
            __builtin_memcpy(&w[q], p + t, 16);
        } else {
            float f[V];
#pragma unroll
            for (int e = 0; e < V; ++e) f[e] = t + e < L ? E::load1(p, t + e) : 0.0f;
            w[q] = E::pack(f);  // exact: the values came from this storage type
        }
    }
}

// B or C of one tile: lanes 0..31 load B, 32..63 load C, four steps of one state each.
template <bool VEC>
__device__ __forceinline__ void load_bc(const BwdArgs& a, int64_t t0, float (&bc)[4]) {
    const int lane = threadIdx.x;
    const int half = lane & 1;
    const int n = (lane >> 1) & (kN - 1);
    const float* src = (lane >= 32 ? a.C : a.B) + ((int64_t)blockIdx.y * kN + n) * a.L;
    const int64_t tb = t0 + 4 * half;
    if (VEC) {  // always issued (past the end from an in-range address, then zeroed): no branch
        const bool in = tb < a.L;
        const float4 v = *reinterpret_cast<const float4*>(src + (in ? tb : a.L - 4));
        bc[0] = in ? v.x : 0.0f; bc[1] = in ? v.y : 0.0f; bc[2] = in ? v.z : 0.0f; bc[3] = in ? v.w : 0.0f;
    } else if (tb + 4 <= a.L) {  // rows of any length: an element-aligned 16-byte load
        __builtin_memcpy(bc, src + tb, 16);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) bc[e] = (tb + e < a.L) ? src[tb + e] : 0.0f;
    }
}

template <class E, bool VEC, bool HAS_Z>
__device__ __forceinline__ void load_raw(const BwdArgs& a, const Row& r, int64_t t0, Raw<E, VEC>& w) {
    const int64_t off = r.row * a.L;
    raw_row<E, VEC>(a.u, off, t0, a.L, w.u);
    raw_row<E, VEC>(a.delta, off, t0, a.L, w.d);
    raw_row<E, VEC>(a.dout, off, t0, a.L, w.g);
    if (HAS_Z) raw_row<E, VEC>(a.z, off, t0, a.L, w.z);
    load_bc<VEC>(a, t0, w.bc);
}

// The tile's B | C block into LDS, time-major: sbc[t][n] = B, sbc[t][16 + n] = C.  Steps at or
// past the batch's length stage as zeros: whatever the tensors hold there cannot reach a sum.
__device__ __forceinline__ void put_bc(const float (&bc)[4], float* sbc, int64_t t0, int64_t stop) {
    const int lane = threadIdx.x;
    const int half = lane & 1;
    const int col = (lane >= 32 ? kN : 0) + ((lane >> 1) & (kN - 1));
#pragma unroll
    for (int e = 0; e < 4; ++e) sbc[(4 * half + e) * kBCs + col] = t0 + 4 * half + e < stop ? bc[e] : 0.0f;
}

// Per-step scalars of one lane.  Inactive lanes and steps past L get dt = x = dy = 0, which
// makes their steps identities and their dB / dC terms exact zeros.
struct StepVals {
    float dt[kBT], x[kBT], dsp[kBT], dy[kBT], dg[kBT], u[kBT];
};

template <class E, bool VEC, bool SOFTPLUS, bool HAS_Z>
__device__ __forceinline__ void step_vals(const BwdArgs& a, const Row& r, int64_t t0, const Raw<E, VEC>& w,
                                          StepVals& s) {
    float dv[kBT], gv[kBT], zv[kBT];
    constexpr int V = E::kPerVec;
#pragma unroll
    for (int q = 0; q < Raw<E, true>::NV; ++q) {
        E::unpack(w.u[q], &s.u[q * V]);
        E::unpack(w.d[q], &dv[q * V]);
        E::unpack(w.g[q], &gv[q * V]);
        if (HAS_Z) E::unpack(w.z[q], &zv[q * V]);
    }
#pragma unroll
    for (int j = 0; j < kBT; ++j) {
        const bool ok = r.active && t0 + j < r.stop;  // past the end: an identity step, no output
        const float pre = dv[j] + r.bias;
        const float dt = SOFTPLUS ? softplus(pre) : pre;
        s.dt[j] = ok ? dt : 0.0f;
        s.dsp[j] = SOFTPLUS ? sigmoid(pre) : 1.0f;
        s.u[j] = ok ? s.u[j] : 0.0f;
        s.x[j] = s.dt[j] * s.u[j];
        if (HAS_Z) {
            const float zz = zv[j];
            const float sg = sigmoid(zz);
            s.dy[j] = ok ? gv[j] * zz * sg : 0.0f;
            s.dg[j] = gv[j] * sg * fmaf(zz, 1.0f - sg, 1.0f);
        } else {
            s.dy[j] = ok ? gv[j] : 0.0f;
            s.dg[j] = 0.0f;
        }
    }
}

__device__ __forceinline__ void seg_tiles(int s, int S, int64_t ntiles, int64_t& tb, int64_t& te) {
    tb = (int64_t)s * ntiles / S;
    te = (int64_t)(s + 1) * ntiles / S;
}

// ---------------------------------------------------------------- aggregate kernel

// The workgroup is one wavefront, whose LDS instructions execute in issue order: ordering LDS
// accesses between its lanes only needs the compiler to keep them in program order.  A
// workgroup barrier would also wait for the global-to-LDS loads in flight.
__device__ __forceinline__ void wave_lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// All of the wave's LDS reads have returned (s_waitcnt lgkmcnt(0), other counters untouched).
__device__ __forceinline__ void lds_reads_done() {
    wave_lds_order();
    __builtin_amdgcn_s_waitcnt(0xC07F);
}

// The aggregate walk, shared by both ways of fetching the inputs: per tile the checkpoint, then
// the recurrences of H (the state from h = 0), Rp (the product of abar since the segment start)
// and Lam (the adjoint carry).
struct AggState {
    float H[kN], Lam[kN], Rp[kN];  // Rp: the power path keeps only Rp[0]
    float dsum;
};

// The tile's start state from h = 0 at the segment start, and sum dt.  ALL: every lane stores
// (see agg_body_staged), else only the active ones.
template <bool ALL>
__device__ __forceinline__ void agg_checkpoint(const BwdArgs& a, const Row& r, int64_t tile, const AggState& st) {
    if (ALL || r.active) {
        float* ck = a.ck + tile * kCkW * a.R + r.row;
#pragma unroll
        for (int n = 0; n < kN; ++n, ck += a.R) *ck = st.H[n];
        *ck = st.dsum;
    }
}

// SAVED: the forward saved the states, so only the adjoint carry (and sum dt) is walked.
template <bool POW, bool SAVED>
__device__ __forceinline__ void agg_tile(const BwdArgs& a, const Row& r, int64_t t0, const StepVals& v,
                                         const float* sbc, AggState& st) {
#pragma unroll
    for (int j = 0; j < kBT; ++j) {
        if (t0 + j >= a.L) break;
        float bv[kN], cv[kN], p[kN];
        read_bc(sbc, j, bv, cv);
        abar16<POW>(v.dt[j], r.A2, p);
        st.dsum += v.dt[j];
#pragma unroll
        for (int n = 0; n < kN; ++n)
            if (!SAVED) st.H[n] = fmaf(p[n], st.H[n], v.x[j] * bv[n]);
        if (POW) {
            // the product of abar_n since the segment start is R^(n+1), R that of abar_0: the
            // weights dy R^(n+1) come from four interleaved chains stepping by R^4
            st.Rp[0] *= p[0];
            const float R = st.Rp[0], R2 = R * R, R4 = R2 * R2;
            float q[4] = {v.dy[j] * R, v.dy[j] * R2, v.dy[j] * (R2 * R), v.dy[j] * R4};
#pragma unroll
            for (int n = 0; n < kN; n += 4) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    st.Lam[n + i] = fmaf(q[i], cv[n + i], st.Lam[n + i]);
                    if (n + 4 < kN) q[i] *= R4;
                }
            }
        } else {
#pragma unroll
            for (int n = 0; n < kN; ++n) {
                st.Rp[n] *= p[n];
                st.Lam[n] = fmaf(st.Rp[n], v.dy[j] * cv[n], st.Lam[n]);
            }
        }
    }
}

template <bool ALL>
__device__ __forceinline__ void agg_finish(const BwdArgs& a, const Row& r, int s, const AggState& st) {
    if (ALL || r.active) {
        float* o = a.agg + (int64_t)s * kAggW * a.R + r.row;
        o[0] = st.dsum;
#pragma unroll
        for (int n = 0; n < kN; ++n) {
            o[(int64_t)(1 + n) * a.R] = st.H[n];
            o[(int64_t)(1 + kN + n) * a.R] = st.Lam[n];
        }
    }
}

__device__ __forceinline__ void agg_init(AggState& st) {
#pragma unroll
    for (int n = 0; n < kN; ++n) { st.H[n] = 0.0f; st.Lam[n] = 0.0f; st.Rp[n] = 1.0f; }
    st.dsum = 0.0f;
}

// Each tile's inputs come straight into registers, one tile ahead (any layout; rows of whole
// 16-byte vectors use the staged variant below).
template <class E, bool VEC, bool SOFTPLUS, bool HAS_Z, bool POW, bool SAVED>
__device__ __forceinline__ void agg_body(const BwdArgs& a, const Row& r, float* sbc) {
    const int s = blockIdx.z;
    int64_t tb, te;
    seg_tiles(s, a.S, a.ntiles, tb, te);
    AggState st;
    agg_init(st);
    Raw<E, VEC> nx;
    load_raw<E, VEC, HAS_Z>(a, r, tb * kBT, nx);
    for (int64_t tile = tb; tile < te; ++tile) {
        const int64_t t0 = tile * kBT;
        if (!SAVED) agg_checkpoint<false>(a, r, tile, st);
        const Raw<E, VEC> cur = nx;
        if (tile + 1 < te) load_raw<E, VEC, HAS_Z>(a, r, t0 + kBT, nx);
        StepVals v;
        step_vals<E, VEC, SOFTPLUS, HAS_Z>(a, r, t0, cur, v);
        wave_lds_order();  // after the previous tile's reads of the B / C block
        put_bc(cur.bc, sbc, t0, r.stop);
        wave_lds_order();
        agg_tile<POW, SAVED>(a, r, t0, v, sbc, st);
    }
    agg_finish<false>(a, r, s, st);
}

// Rows of whole 16-byte vectors: the inputs are fetched a block at a time, 64 bytes of every row
// and array (half a 128-byte line), by global-to-LDS loads issued together.  Loading 16 bytes
// per row per tile instead spreads the reads of one line over eight tiles; with all rows of
// all wavefronts in flight the line leaves the L2 in between and is fetched again each time.
// The block sits in LDS as [array][chunk][lane] 16-byte words (a lane reads back only what it
// loaded: its own row).  The next block is requested once the current block's last tile has been
// read into registers, so its latency overlaps that tile's arithmetic.
// 16 bytes per lane from global memory into LDS: lane l's bytes land at dst + 16 l (dst is the
// same for the whole wave).
__device__ __forceinline__ void lds_load16(const void* src, uint4* dst) {
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

constexpr int kStageChunks = 4;  // 16-byte chunks per row and array in one block

template <class E>
struct StageGeo {
    static constexpr int V = E::kPerVec;              // steps per chunk
    static constexpr int NV = kBT / V;                // chunks per tile
    static constexpr int TPB = kStageChunks / NV;     // tiles per block
};

// SAVED: u is not read (it only feeds the forward state, which the forward saved).
template <class E, bool HAS_Z, bool SAVED>
__device__ __forceinline__ void stage_block(const BwdArgs& a, const Row& r, int64_t tile, uint4* stage) {
    using G = StageGeo<E>;
    using S_t = typename E::storage;
    const int64_t off = r.row * a.L;
    const void* src[4] = {a.u, a.delta, a.dout, a.z};
#pragma unroll
    for (int c = 0; c < kStageChunks; ++c) {
        const int64_t t = tile * kBT + c * G::V;
        const int64_t tc = t < a.L ? t : 0;  // past the row's end: any valid address, those steps are masked
#pragma unroll
        for (int q = SAVED ? 1 : 0; q < (HAS_Z ? 4 : 3); ++q)
            lds_load16(static_cast<const S_t*>(src[q]) + off + tc, stage + (q * kStageChunks + c) * 64);
    }
}

template <class E, bool HAS_Z>
__device__ __forceinline__ void staged_tile(const uint4* stage, int k, Raw<E, true>& w) {
    using G = StageGeo<E>;
    const int lane = threadIdx.x;
#pragma unroll
    for (int q = 0; q < G::NV; ++q) {
        const int c = k * G::NV + q;
        w.u[q] = stage[(0 * kStageChunks + c) * 64 + lane];
        w.d[q] = stage[(1 * kStageChunks + c) * 64 + lane];
        w.g[q] = stage[(2 * kStageChunks + c) * 64 + lane];
        if (HAS_Z) w.z[q] = stage[(3 * kStageChunks + c) * 64 + lane];
    }
}

// Lanes past the last channel (a partial channel group) read the last channel's row (their row
// index is clamped to it); here they also compute its values, so every lane stores and a
// duplicate writes the same bits as the owner.  Stores without a branch keep the count of
// outstanding memory operations exact, so waiting for the next tile's B / C does not also wait
// for the block in flight.
template <class E, bool SOFTPLUS, bool HAS_Z, bool POW, bool SAVED>
__device__ __forceinline__ void agg_body_staged(const BwdArgs& a, const Row& r_in, float* sbc, uint4* stage) {
    using G = StageGeo<E>;
    Row r = r_in;
    r.active = true;
    const int s = blockIdx.z;
    int64_t tb, te;
    seg_tiles(s, a.S, a.ntiles, tb, te);
    AggState st;
    agg_init(st);
    float bc_next[4];
    stage_block<E, HAS_Z, SAVED>(a, r, tb, stage);
    load_bc<true>(a, tb * kBT, bc_next);
    for (int64_t blk = tb; blk < te; blk += G::TPB) {
        // the block's tiles, unrolled: a tile's LDS words are read one tile ahead, and the
        // next block is requested before the last tile's arithmetic
        Raw<E, true> cur;
        staged_tile<E, HAS_Z>(stage, 0, cur);
#pragma unroll
        for (int k = 0; k < G::TPB; ++k) {
            const int64_t tile = blk + k;
            if (tile >= te) break;
            const int64_t t0 = tile * kBT;
            // B / C of the next tile are requested before this tile's checkpoint stores, so
            // waiting for them later does not wait for the stores
#pragma unroll
            for (int e = 0; e < 4; ++e) cur.bc[e] = bc_next[e];
            load_bc<true>(a, t0 + kBT, bc_next);
            if (!SAVED) agg_checkpoint<true>(a, r, tile, st);
            Raw<E, true> nx;
            if (k + 1 < G::TPB) {
                staged_tile<E, HAS_Z>(stage, k + 1, nx);
            } else if (tile + 1 < te) {
                lds_reads_done();  // the block's LDS reads are complete before it is overwritten
                stage_block<E, HAS_Z, SAVED>(a, r, tile + 1, stage);
            }
            StepVals v;
            step_vals<E, true, SOFTPLUS, HAS_Z>(a, r, t0, cur, v);
            wave_lds_order();  // after the previous tile's reads of the B / C block
            put_bc(cur.bc, sbc, t0, r.stop);
            wave_lds_order();
            agg_tile<POW, SAVED>(a, r, t0, v, sbc, st);
            if (k + 1 < G::TPB) cur = nx;
        }
    }
    agg_finish<true>(a, r, s, st);
}

template <class E, bool VEC, bool SOFTPLUS, bool HAS_Z, bool SAVED>
__global__ __launch_bounds__(64) void bwd_agg_kernel(BwdArgs a) {
    __shared__ __align__(16) float sbc[kBT * kBCs];
    const Row r = row_of(a);
    if constexpr (VEC) {
        __shared__ __align__(16) uint4 stage[4 * kStageChunks * 64];
        if (__all(r.pow_ok)) agg_body_staged<E, SOFTPLUS, HAS_Z, true, SAVED>(a, r, sbc, stage);
        else agg_body_staged<E, SOFTPLUS, HAS_Z, false, SAVED>(a, r, sbc, stage);
    } else {
        if (__all(r.pow_ok)) agg_body<E, VEC, SOFTPLUS, HAS_Z, true, SAVED>(a, r, sbc);
        else agg_body<E, VEC, SOFTPLUS, HAS_Z, false, SAVED>(a, r, sbc);
    }
}

// ---------------------------------------------------------------- main kernel

// Segment carries: the forward state entering segment s (fold of segments 0..s-1) and the
// adjoint entering its last step from the later segments (fold of S-1 down to s+1).
// WITH_H: also the forward state (not needed when the forward saved its states).
template <bool POW, bool WITH_H>
__device__ __forceinline__ void carries(const BwdArgs& a, const Row& r, int s, float (&h)[kN],
                                        float (&gc)[kN]) {
#pragma unroll
    for (int n = 0; n < kN; ++n) {
        h[n] = a.h0 ? a.h0[r.row * kN + n] : 0.0f;        // the forward's starting state
        gc[n] = a.dlast ? a.dlast[r.row * kN + n] : 0.0f; // dL/dh at the last step, if any
    }
    for (int k = 0; k < (WITH_H ? s : 0); ++k) {
        const float* g = a.agg + (int64_t)k * kAggW * a.R + r.row;
        float p[kN];
        abar16<POW>(g[0], r.A2, p);
#pragma unroll
        for (int n = 0; n < kN; ++n) h[n] = fmaf(p[n], h[n], g[(int64_t)(1 + n) * a.R]);
    }
    for (int k = a.S - 1; k > s; --k) {
        const float* g = a.agg + (int64_t)k * kAggW * a.R + r.row;
        float p[kN];
        abar16<POW>(g[0], r.A2, p);
#pragma unroll
        for (int n = 0; n < kN; ++n) gc[n] = fmaf(p[n], gc[n], g[(int64_t)(1 + kN + n) * a.R]);
    }
}

template <class E, bool VEC, bool SOFTPLUS, bool HAS_Z, bool POW, bool SAVED>
__device__ __forceinline__ void main_body(const BwdArgs& a, const Row& r, float* sbc, float* hbuf,
                                          float* hin) {
    const int s = blockIdx.z;
    const int lane = threadIdx.x;
    const int b = blockIdx.y;
    int64_t tb, te;
    seg_tiles(s, a.S, a.ntiles, tb, te);
    float h[kN], gc[kN];  // state entering the segment; adjoint entering its last step
    carries<POW, !SAVED>(a, r, s, h, gc);

    // backward walk
    float dA[kN];
#pragma unroll
    for (int n = 0; n < kN; ++n) dA[n] = 0.0f;
    float dDacc = 0.0f, dbacc = 0.0f;
    Raw<E, VEC> nx;
    load_raw<E, VEC, HAS_Z>(a, r, (te - 1) * kBT, nx);
    if (!SAVED) {
#pragma unroll
        for (int n = 0; n < kN; ++n) hin[n * 64 + lane] = h[n];  // h_in waits in LDS: fewer live VGPRs
    }
    for (int64_t tile = te - 1; tile >= tb; --tile) {
        const int64_t t0 = tile * kBT;
        const Raw<E, VEC> cur = nx;
        float ck0[kCkW];  // loaded here, used after the tile's set-up (SAVED: the true start state)
        if (SAVED) {
            const float4* sp = reinterpret_cast<const float4*>(a.saved + tile * kN * a.R + r.row * 4);
#pragma unroll
            for (int q = 0; q < kN / 4; ++q) {
                const float4 v = r.active ? sp[q * a.R] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                ck0[4 * q] = v.x; ck0[4 * q + 1] = v.y; ck0[4 * q + 2] = v.z; ck0[4 * q + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int n = 0; n < kCkW; ++n) ck0[n] = r.active ? a.ck[(tile * kCkW + n) * a.R + r.row] : 0.0f;
        }
        if (tile > tb) load_raw<E, VEC, HAS_Z>(a, r, t0 - kBT, nx);
        StepVals v;
        step_vals<E, VEC, SOFTPLUS, HAS_Z>(a, r, t0, cur, v);
        float a0[kBT];  // abar_0 of each step (power path)
#pragma unroll
        for (int j = 0; j < kBT; ++j) a0[j] = POW ? fast_exp2(v.dt[j] * r.A2[0]) : 0.0f;
        wave_lds_order();  // after the previous tile's reads of the B / C block
        put_bc(cur.bc, sbc, t0, r.stop);
        wave_lds_order();
        // The tile's 16 states in two halves of 8 (the states are independent in the recurrence;
        // only the outputs' sums over n combine the halves): recompute the half's states from
        // the checkpoint into LDS (lane-private columns), then consume them in reverse.
        float yacc[kBT], gbacc[kBT], qaacc[kBT];
#pragma unroll
        for (int j = 0; j < kBT; ++j) yacc[j] = gbacc[j] = qaacc[j] = 0.0f;
        constexpr int kQ = q_steps<E>();
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            float pc[kH];  // tile start: exp(A sum dt) h_in + the local checkpoint (SAVED: given)
            if (!SAVED) abar8<POW>(ck0[kN], POW ? fast_exp2(ck0[kN] * r.A2[0]) : 0.0f, r.A2, hf, pc);
            float bcs[kBT];
            // Steps in chunks of kQ, the latest first: each chunk recomputes the half's states from
            // the tile start, keeps its own steps' states in LDS and consumes them in reverse (a
            // later chunk walks the earlier steps too; LDS holds kQ steps, not kBT).
#pragma unroll
            for (int c = kBT / kQ - 1; c >= 0; --c) {
                float hs[kH];
#pragma unroll
                for (int k = 0; k < kH; ++k)
                    hs[k] = SAVED ? ck0[kH * hf + k] : fmaf(pc[k], hin[(kH * hf + k) * 64 + lane], ck0[kH * hf + k]);
#pragma unroll
                for (int j = 0; j < kQ * (c + 1); ++j) {
                    if (t0 + j >= a.L) break;
                    float bv[kH], cv[kH], p[kH];
                    read_bc_half(sbc, j, hf, bv, cv);
                    abar8<POW>(v.dt[j], a0[j], r.A2, hf, p);
#pragma unroll
                    for (int k = 0; k < kH; ++k) {
                        hs[k] = fmaf(p[k], hs[k], v.x[j] * bv[k]);
                        if (j >= kQ * c) hbuf[((j - kQ * c) * kH + k) * 64 + lane] = hs[k];
                    }
                }
#pragma unroll
                for (int j = kQ * (c + 1) - 1; j >= kQ * c; --j) {
                    bcs[j] = 0.0f;
                    if (t0 + j >= a.L) continue;
                    float bv[kH], cv[kH], p[kH], hc[kH];
                    read_bc_half(sbc, j, hf, bv, cv);
                    abar8<POW>(v.dt[j], a0[j], r.A2, hf, p);
#pragma unroll
                    for (int k = 0; k < kH; ++k) hc[k] = hbuf[((j - kQ * c) * kH + k) * 64 + lane];
                    float y = 0.0f, gb = 0.0f, qa = 0.0f, tm[2 * kH];
#pragma unroll
                    for (int k = 0; k < kH; ++k) {
                        const int n = kH * hf + k;
                        const float G = fmaf(v.dy[j], cv[k], gc[n]);       // dL/dh_t
                        y = fmaf(cv[k], hc[k], y);
                        const float ah = fmaf(-v.x[j], bv[k], hc[k]);      // abar h_{t-1}
                        const float qn = G * ah;
                        qa = fmaf(POW ? static_cast<float>(n + 1) : r.An[n], qn, qa);
                        gb = fmaf(G, bv[k], gb);
                        dA[n] = fmaf(v.dt[j], qn, dA[n]);
                        tm[k] = G * v.x[j];                                // dB term
                        tm[kH + k] = v.dy[j] * hc[k];                      // dC term
                        gc[n] = p[k] * G;                                  // toward h_{t-1}
                    }
                    yacc[j] += y;
                    gbacc[j] += gb;
                    qaacc[j] += qa;
                    bcs[j] = lanes_sum16(tm);  // over the wave's 64 channels
                }
            }
            if ((lane & 3) == 0) {  // one lane per term: dB of state kH hf + k, or dC of state kH hf + k - kH
                const int k = sum16_term(lane);
                const int idx = k < kH ? kH * hf + k : kN + kH * hf + (k - kH);
                float4* o = reinterpret_cast<float4*>(
                    a.part + (((int64_t)blockIdx.x * a.Bt + b) * (2 * kN) + idx) * a.tpad + t0);
                o[0] = make_float4(bcs[0], bcs[1], bcs[2], bcs[3]);
                o[1] = make_float4(bcs[4], bcs[5], bcs[6], bcs[7]);
            }
        }
        float gdu[kBT], gdd[kBT], gdz[kBT];
#pragma unroll
        for (int j = 0; j < kBT; ++j) {
            const float qa = POW ? qaacc[j] * r.An[0] : qaacc[j];
            gdu[j] = fmaf(v.dt[j], gbacc[j], r.dskip * v.dy[j]);
            gdd[j] = fmaf(v.u[j], gbacc[j], qa) * v.dsp[j];
            gdz[j] = v.dg[j] * fmaf(r.dskip, v.u[j], yacc[j]);
            if (t0 + j >= r.stop) gdu[j] = gdd[j] = gdz[j] = 0.0f;  // past the sequence's end
            if (t0 + j < a.L) {
                dDacc = fmaf(v.dy[j], v.u[j], dDacc);
                dbacc += r.active ? gdd[j] : 0.0f;
            }
        }
        if (r.active) {
            const int64_t off = r.row * a.L;
            store_tile<E, VEC>(a.du, off, t0, a.L, gdu);
            store_tile<E, VEC>(a.ddelta, off, t0, a.L, gdd);
            if (HAS_Z && a.dz) store_tile<E, VEC>(a.dz, off, t0, a.L, gdz);
        }
    }
    if (r.active) {
        float* o = a.par + (int64_t)s * kParW * a.R + r.row;
#pragma unroll
        for (int n = 0; n < kN; ++n) o[(int64_t)n * a.R] = dA[n];
        o[(int64_t)kN * a.R] = dDacc;
        o[(int64_t)(kN + 1) * a.R] = dbacc;
    }
    if (a.dh0 && r.active && s == 0) {  // what flows out of step 0: dL/dh0
#pragma unroll
        for (int n = 0; n < kN; ++n) a.dh0[r.row * kN + n] = gc[n];
    }
}

template <class E, bool VEC, bool SOFTPLUS, bool HAS_Z, bool SAVED>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void bwd_main_kernel(BwdArgs a) {
    __shared__ __align__(16) float sbc[kBT * kBCs];
    __shared__ __align__(16) float hbuf[q_steps<E>() * kH * 64];
    __shared__ __align__(16) float hin[kN * 64];
    const Row r = row_of(a);
    if (__all(r.pow_ok)) main_body<E, VEC, SOFTPLUS, HAS_Z, true, SAVED>(a, r, sbc, hbuf, hin);
    else main_body<E, VEC, SOFTPLUS, HAS_Z, false, SAVED>(a, r, sbc, hbuf, hin);
}

// ---------------------------------------------------------------- reductions

// dB[b][n][t] = sum_g part[g][b][n][t], dC[b][n][t] = sum_g part[g][b][16 + n][t].
// Each lane sums kRedV consecutive steps of one (b, k) over the G groups, in group order (the
// same order for every call), with kRedU groups' loads in flight; the partial rows are padded to
// a multiple of kBT steps, so the vector loads stay inside them.
constexpr int kRedV = 4, kRedU = 8;
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(const float* __restrict__ part, float* __restrict__ dB,
                                                            float* __restrict__ dC, int G, int Bt, int64_t L,
                                                            int64_t tpad) {
    const int64_t nv = tpad / kRedV;                 // vectors per padded row
    const int64_t total = (int64_t)Bt * 2 * kN * nv;
    const int64_t gstride = (int64_t)Bt * 2 * kN * tpad / kRedV;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t v = i % nv;
        const int64_t bk = i / nv;           // b * 32 + k
        const int64_t t = v * kRedV;
        if (t >= L) continue;                // padding only
        const int k = static_cast<int>(bk % (2 * kN));
        const int64_t b = bk / (2 * kN);
        const float4* p = reinterpret_cast<const float4*>(part) + bk * nv + v;
        float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll kRedU
        for (int g = 0; g < G; ++g) {
            const float4 q = p[(int64_t)g * gstride];
            s.x += q.x; s.y += q.y; s.z += q.z; s.w += q.w;
        }
        float* dst = k < kN ? dB + (b * kN + k) * L : dC + (b * kN + (k - kN)) * L;
        const float o[kRedV] = {s.x, s.y, s.z, s.w};
#pragma unroll
        for (int e = 0; e < kRedV; ++e)
            if (t + e < L) dst[t + e] = o[e];
    }
}

// dA[d][n], dD[d], dbias[d]: sums of the per-(segment, row) partials over segments and batches.
__global__ __launch_bounds__(256) void bwd_reduce_par_kernel(const float* __restrict__ par, float* __restrict__ dA,
                                                             float* __restrict__ dD, float* __restrict__ dbias,
                                                             int S, int Bt, int64_t Dn, int64_t R) {
    const int64_t total = (int64_t)kParW * Dn;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int k = static_cast<int>(i / Dn);
        const int64_t d = i % Dn;
        float s = 0.0f;  // segment-major, batch-minor order, kRedU loads in flight
        const int n = S * Bt;
#pragma unroll kRedU
        for (int j = 0; j < n; ++j) {
            const int sg = j / Bt, b = j - sg * Bt;
            s += par[((int64_t)sg * kParW + k) * R + (int64_t)b * Dn + d];
        }
        if (k < kN) dA[d * kN + k] = s;
        else if (k == kN) { if (dD) dD[d] = s; }
        else if (dbias) dbias[d] = s;
    }
}

__global__ __launch_bounds__(256) void bwd_zero_kernel(float* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.0f;
}

unsigned grid_for(int64_t n) {
    const int64_t b = (n + 255) / 256;
    return static_cast<unsigned>(b < 1 ? 1 : (b > 65535 ? 65535 : b));
}

hipError_t zero(float* p, int64_t n, hipStream_t s) {
    if (!p || n <= 0) return hipSuccess;
    bwd_zero_kernel<<<dim3(grid_for(n)), dim3(256), 0, s>>>(p, n);
    return hipGetLastError();
}

template <class E, bool VEC, bool SOFTPLUS, bool HAS_Z>
hipError_t launch_t(const BwdArgs& k, const BwdLaunch& a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(k.G), static_cast<unsigned>(k.Bt), static_cast<unsigned>(k.S));
    if (k.saved) {
        bwd_agg_kernel<E, VEC, SOFTPLUS, HAS_Z, true><<<grid, dim3(64), 0, stream>>>(k);
        bwd_main_kernel<E, VEC, SOFTPLUS, HAS_Z, true><<<grid, dim3(64), 0, stream>>>(k);
    } else {
        bwd_agg_kernel<E, VEC, SOFTPLUS, HAS_Z, false><<<grid, dim3(64), 0, stream>>>(k);
        bwd_main_kernel<E, VEC, SOFTPLUS, HAS_Z, false><<<grid, dim3(64), 0, stream>>>(k);
    }
    const int64_t nbc = (int64_t)k.Bt * 2 * kN * (k.tpad / kRedV);
    bwd_reduce_bc_kernel<<<dim3(grid_for(nbc)), dim3(256), 0, stream>>>(k.part, a.dB, a.dC, k.G, k.Bt, k.L, k.tpad);
    bwd_reduce_par_kernel<<<dim3(grid_for((int64_t)kParW * k.Dn)), dim3(256), 0, stream>>>(
        k.par, a.dA, a.dD, a.dbias, k.S, k.Bt, k.Dn, k.R);
    return hipGetLastError();
}

template <class E, bool VEC>
hipError_t launch_e(const BwdArgs& k, const BwdLaunch& a, hipStream_t stream) {
    const bool hz = a.z != nullptr;
    if (a.softplus) return hz ? launch_t<E, VEC, true, true>(k, a, stream) : launch_t<E, VEC, true, false>(k, a, stream);
    return hz ? launch_t<E, VEC, false, true>(k, a, stream) : launch_t<E, VEC, false, false>(k, a, stream);
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct Layout {
    size_t agg, ck, part, par, total;
};

Layout layout_of(const BwdLaunch& a, int S) {  // no checkpoints when the forward saved its states
    const int64_t R = a.Bt * a.Dn;
    const int64_t ntiles = (a.L + kBT - 1) / kBT;
    const int64_t G = (a.Dn + 63) / 64;
    Layout l;
    l.agg = 0;
    l.ck = l.agg + align256(static_cast<size_t>(S) * kAggW * R * sizeof(float));
    l.part = l.ck + (a.saved ? 0 : align256(static_cast<size_t>(ntiles) * kCkW * R * sizeof(float)));
    l.par = l.part + align256(static_cast<size_t>(G) * a.Bt * 2 * kN * ntiles * kBT * sizeof(float));
    l.total = l.par + align256(static_cast<size_t>(S) * kParW * R * sizeof(float));
    return l;
}

}  // namespace

// Segments per channel group: as many wavefronts as fit on the chip at once (the main kernel's
// LDS and 256 VGPRs allow eight per CU for bf16 rows, seven for fp32 rows), at most one per tile.
// `segments_override` > 0 replaces the count (tests force many or few segments with it).
int plan_bwd_segments(const BwdLaunch& a, int num_cus, int segments_override) {
    const int64_t groups = a.Bt * ((a.Dn + 63) / 64);
    const int64_t ntiles = (a.L + kBT - 1) / kBT;
    const int64_t target = (a.bf16 ? 8LL : 7LL) * (num_cus > 0 ? num_cus : 256);
    int64_t S = groups > 0 ? target / groups : 1;  // one round: every wavefront resident at once
    if (segments_override > 0) S = segments_override;
    if (S > ntiles) S = ntiles;
    if (S > 65535) S = 65535;
    if (S < 1) S = 1;
    return static_cast<int>(S);
}

size_t bwd_workspace_bytes(const BwdLaunch& a, int segments) {
    if (a.L == 0 || a.Bt * a.Dn == 0) return 0;
    return layout_of(a, segments).total;
}

hipError_t launch_scan_bwd(const BwdLaunch& a, int segments, void* workspace, hipStream_t stream) {
    const int64_t R = a.Bt * a.Dn;
    if (a.L == 0 || R == 0) {
        // empty sums: every reduced gradient is zero (du / ddelta / dz have no elements), and
        // dL/dh0 is dL/d last_state
        hipError_t e = zero(a.dA, a.Dn * kN, stream);
        if (e == hipSuccess && a.dh0 && R > 0) {
            if (a.dlast) e = hipMemcpyAsync(a.dh0, a.dlast, R * kN * sizeof(float), hipMemcpyDeviceToDevice, stream);
            else e = zero(a.dh0, R * kN, stream);
        }
        if (e == hipSuccess) e = zero(a.dD, a.Dn, stream);
        if (e == hipSuccess) e = zero(a.dbias, a.Dn, stream);
        if (e == hipSuccess) e = zero(a.dB, a.Bt * kN * a.L, stream);
        if (e == hipSuccess) e = zero(a.dC, a.Bt * kN * a.L, stream);
        return e;
    }
    const Layout l = layout_of(a, segments);
    char* ws = static_cast<char*>(workspace);
    BwdArgs k;
    k.u = a.u; k.delta = a.delta; k.z = a.z; k.dout = a.dout;
    k.A = a.A; k.B = a.B; k.C = a.C; k.D = a.D; k.bias = a.bias;
    k.du = a.du; k.ddelta = a.ddelta; k.dz = a.dz;
    k.h0 = a.h0; k.lens = a.lens; k.dlast = a.dlast; k.dh0 = a.dh0; k.saved = a.saved;
    k.agg = reinterpret_cast<float*>(ws + l.agg);
    k.ck = reinterpret_cast<float*>(ws + l.ck);
    k.part = reinterpret_cast<float*>(ws + l.part);
    k.par = reinterpret_cast<float*>(ws + l.par);
    k.Dn = a.Dn; k.L = a.L; k.R = R;
    k.ntiles = (a.L + kBT - 1) / kBT;
    k.tpad = k.ntiles * kBT;
    k.S = segments;
    k.G = static_cast<int>((a.Dn + 63) / 64);
    k.Bt = static_cast<int>(a.Bt);
    if (a.bf16) return a.vec_ok ? launch_e<BF16, true>(k, a, stream) : launch_e<BF16, false>(k, a, stream);
    return a.vec_ok ? launch_e<F32, true>(k, a, stream) : launch_e<F32, false>(k, a, stream);
}

}  // namespace mss
