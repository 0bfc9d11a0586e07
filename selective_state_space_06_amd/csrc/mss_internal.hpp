// mss_internal.hpp -- host-side launch descriptions passed from the validated C ABI
// (abi.hip) to the kernel launchers (scan_fwd.hip, state_update.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mss {

constexpr int kN = 16;      // d_state handled by the kernels
constexpr int kRows = 64;   // channels per wavefront (one lane per channel)
// Bytes of each row (per array) a fast-path tile covers: 64 for bf16 rows (half a 128-byte line:
// the LDS of two wavefronts per SIMD holds no more), a whole line for fp32 rows (one wavefront per
// SIMD leaves the LDS for it, and each line is then fetched once).
constexpr int fast_tile_bytes(bool bf16) { return bf16 ? 64 : 128; }

struct ScanLaunch {
    const void* u;
    const void* delta;
    const void* z;          // nullable
    const float* A;         // (Dn, N)
    const float* B;         // (Bt, N, L)
    const float* C;         // (Bt, N, L)
    const float* D;         // nullable
    const float* bias;      // nullable
    void* out;
    float* last_state;      // nullable
    const float* h0;        // nullable: starting state (Bt, Dn, N), zeros when null
    const int32_t* lens;    // nullable: per-batch sequence lengths (device), clamped to [0, L]
    float* saved;           // nullable: the state entering every 8-step tile, [ceil(L/8)][N][Bt*Dn]
    int64_t Bt, Dn, L;
    int N = 16;             // d_state: 16 (fast and general kernels), 32, 64 or 128 (general kernels)
    int softplus;
    bool bf16;              // storage type of u / delta / z / out
    bool vec_ok;            // rows of u / delta / z / out are 16-byte aligned
    // Optional timing events (all null or all valid): recorded on the stream before the first
    // kernel, before the main kernel and after it.
    hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
};

// Records launch-timing event k of `a` on `stream` when timing is on.
inline void mark(const ScanLaunch& a, int k, hipStream_t stream) {
    if (a.ev[k]) (void)hipEventRecord(a.ev[k], stream);
}

struct DecodeLaunch {
    float* state;           // (Bt, Dn, N), in/out
    const void* x;
    const void* dt;
    const void* z;          // nullable
    const float* A;
    const float* B;         // (Bt, N)
    const float* C;         // (Bt, N)
    const float* D;         // nullable
    const float* bias;      // nullable
    void* out;
    int64_t Bt, Dn;
    int N;                  // d_state: 16, 32, 64 or 128
    bool bf16;
};

struct BwdLaunch {
    const void* u;
    const void* delta;
    const void* z;          // nullable
    const void* dout;
    const float* A;
    const float* B;
    const float* C;
    const float* D;         // nullable
    const float* bias;      // nullable
    void* du;
    void* ddelta;
    void* dz;               // nullable (also when z is null)
    float* dA;              // (Dn, N)
    float* dB;              // (Bt, N, L)
    float* dC;              // (Bt, N, L)
    float* dD;              // nullable
    float* dbias;           // nullable
    const float* h0;        // nullable: the forward's starting state (Bt, Dn, N)
    const int32_t* lens;    // nullable: per-batch sequence lengths (device)
    const float* dlast;     // nullable: dL/d last_state (Bt, Dn, N)
    float* dh0;             // nullable: dL/dh0 (Bt, Dn, N), written
    const float* saved;     // nullable: the forward's states entering every 8-step tile
                            // ([ceil(L/8)][N][Bt*Dn]); when given they replace the recomputation
    int64_t Bt, Dn, L;
    int softplus;
    bool bf16;
    bool vec_ok;            // rows of u / delta / z / dout / du / ddelta / dz and B / C 16-byte aligned
};

struct ConvLaunch {
    const void* x;          // (Bt, Dn, L)
    const float* w;         // (Dn, K)
    const float* bias;      // nullable
    const void* state_in;   // (Bt, Dn, K-1), nullable
    void* out;
    void* state_out;        // (Bt, Dn, K-1), nullable
    int64_t Dn, L, R;       // R = Bt * Dn
    int K;
    bool silu, bf16;
    bool vec_ok;            // rows of x / out span whole 16-byte vectors, 16-byte aligned
};

struct ConvUpdateLaunch {
    void* state;            // (Bt, Dn, K-1), in/out
    const void* x;          // (Bt, Dn)
    const float* w;
    const float* bias;
    void* out;
    int64_t Dn, R;
    int K;
    bool silu, bf16;
};

// Mamba-2 SSD layer (ssd_scan.hip): x, z, out (Bt, L, H, P); dt (Bt, L, H); B, C (Bt, L, G, N), all
// bf16; A, D, bias (H) fp32; last_state (Bt, H, P, N) fp32.  P = 64, N = 64 or 128.
struct SsdLaunch {
    const void* x;
    const void* dt;
    const float* A;
    const void* B;
    const void* C;
    const float* D;         // nullable
    const void* z;          // nullable
    const float* bias;      // nullable
    void* out;
    float* last_state;      // nullable
    int64_t Bt, L, H, P, G, N;
    int softplus;
};
// Segments per (batch, head) (segments_override > 0 replaces the count), the workspace they need,
// and the launch.
int plan_ssd_segments(const SsdLaunch& a, int num_cus, int segments_override);
size_t ssd_workspace_bytes(const SsdLaunch& a, int segments);
hipError_t launch_ssd_scan(const SsdLaunch& a, int segments, float* workspace, hipStream_t stream);

// How the forward scan is decomposed.  Generic path: `segments` workgroup-rows per channel
// group, each covering `seg_len` steps.  Fast path: `waves` wavefronts, each taking an equal
// contiguous range of the (channel group, tile) work; `segments` > 1 when some range ends
// inside a group (the aggregate kernel then has work).
struct ScanPlan {
    int segments;
    int64_t seg_len;
    int64_t waves;
    int64_t xcds;            // fast path: XCDs the wavefronts are dealt over
    bool fits = true;        // fast path: the (group, tile) count fits the kernels' 32-bit counts
    size_t workspace_bytes;  // carry workspace needed (0 when nothing is carried)
};

// Segment plan for a time tile of `tile` steps (segments are whole tiles).
ScanPlan plan_scan(const ScanLaunch& a, int num_cus, int tile, int segments_override);
// Generic path (any alignment): scan_fwd.hip.
hipError_t launch_scan_fwd(const ScanLaunch& a, const ScanPlan& plan, float* workspace,
                           hipStream_t stream);
int generic_tile();
size_t generic_workspace_bytes(const ScanLaunch& a, int segments);
// Fast path: scan_fast.hip.  `waves_override` > 0 replaces the automatic wavefront count.
ScanPlan plan_fast(const ScanLaunch& a, int num_cus, int64_t waves_override);
size_t fast_workspace_bytes(const ScanLaunch& a, const ScanPlan& plan);
hipError_t launch_scan_fast(const ScanLaunch& a, const ScanPlan& plan, float* workspace,
                            hipStream_t stream);
hipError_t launch_state_update(const DecodeLaunch& a, hipStream_t stream);
// Causal conv1d: conv1d.hip.
hipError_t launch_conv1d_fwd(const ConvLaunch& a, hipStream_t stream);
hipError_t launch_conv1d_update(const ConvUpdateLaunch& a, hipStream_t stream);
// Backward scan: scan_bwd.hip.
int plan_bwd_segments(const BwdLaunch& a, int num_cus, int segments_override);
size_t bwd_workspace_bytes(const BwdLaunch& a, int segments);
hipError_t launch_scan_bwd(const BwdLaunch& a, int segments, void* workspace, hipStream_t stream);

}  // namespace mss
