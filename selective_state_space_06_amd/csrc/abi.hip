// abi.hip -- the extern "C" boundary of libmamba_scan: argument validation, the carry
// workspace, and dispatch to the gfx950 kernels.  Every check runs before the first HIP call,
// so invalid arguments never reach the device.
#include <atomic>
#include <vector>
#include <initializer_list>
#include <mutex>
#include <thread>
#include <unordered_map>
#include <utility>

#include "mamba_scan.h"
#include "mss_internal.hpp"

namespace {

using mss::kN;

int64_t numel(const mss_tensor_t& t) {
    int64_t n = 1;
    for (int i = 0; i < t.ndim; ++i) n *= t.shape[i];
    return n;
}

size_t elem_size(int32_t dtype) { return dtype == MSS_BF16 ? 2 : 4; }

bool shape_is(const mss_tensor_t& t, int ndim, int64_t s0, int64_t s1 = 0, int64_t s2 = 0, int64_t s3 = 0) {
    if (t.ndim != ndim) return false;
    const int64_t s[4] = {s0, s1, s2, s3};
    for (int i = 0; i < ndim; ++i)
        if (t.shape[i] != s[i]) return false;
    return true;
}

bool dense(const mss_tensor_t& t) {
    if (numel(t) == 0) return true;
    int64_t expect = 1;
    for (int i = t.ndim - 1; i >= 0; --i) {
        if (t.shape[i] != 1 && t.stride[i] != expect) return false;
        expect *= t.shape[i];
    }
    return true;
}

bool aligned(const mss_tensor_t& t, size_t a) {
    return (reinterpret_cast<uintptr_t>(t.data) % a) == 0;
}

struct Range {
    uintptr_t lo, hi;
};
Range range_of(const mss_tensor_t* t) {
    if (!t || !t->data) return {0, 0};
    const uintptr_t lo = reinterpret_cast<uintptr_t>(t->data);
    return {lo, lo + static_cast<uintptr_t>(numel(*t)) * elem_size(t->dtype)};
}
bool overlap(const mss_tensor_t* a, const mss_tensor_t* b) {
    const Range x = range_of(a), y = range_of(b);
    if (x.lo == x.hi || y.lo == y.hi) return false;
    return x.lo < y.hi && y.lo < x.hi;
}

// Status of one descriptor before its extents are compared: NULL descriptor or NULL data
// (for a non-empty tensor) -> NULL_ARG; ndim outside 1..4, a negative extent or an element count
// beyond 2^48 (so that no later size computation can overflow) -> SHAPE.
int check_desc(const mss_tensor_t* t, bool required) {
    if (!t) return required ? MSS_ERR_NULL_ARG : MSS_OK;
    if (t->ndim < 1 || t->ndim > 4) return MSS_ERR_SHAPE;
    int64_t n = 1;
    for (int i = 0; i < t->ndim; ++i) {
        if (t->shape[i] < 0) return MSS_ERR_SHAPE;
        if (__builtin_mul_overflow(n, t->shape[i], &n) || n > (int64_t{1} << 48)) return MSS_ERR_SHAPE;
    }
    if (!t->data && n != 0) return MSS_ERR_NULL_ARG;
    return MSS_OK;
}

template <size_t K>
int check_descs(const mss_tensor_t* const (&req)[K], std::initializer_list<const mss_tensor_t*> opt) {
    for (const mss_tensor_t* t : req)
        if (!t) return MSS_ERR_NULL_ARG;
    for (const mss_tensor_t* t : req) {
        const int s = check_desc(t, true);
        if (s != MSS_OK) return s;
    }
    for (const mss_tensor_t* t : opt) {
        const int s = check_desc(t, false);
        if (s != MSS_OK) return s;
    }
    return MSS_OK;
}

// ---- per-device facts and the per-(device, stream) carry workspace
// hipStreamPerThread is one handle value standing for a different stream in every host thread, so
// its workspaces are also keyed by the calling thread.
struct WsKey {
    int dev;
    void* stream;
    size_t thread;
    bool operator==(const WsKey& o) const { return dev == o.dev && stream == o.stream && thread == o.thread; }
};
struct WsHash {
    size_t operator()(const WsKey& k) const {
        return (std::hash<void*>()(k.stream) * 31u + static_cast<size_t>(k.dev)) * 31u + k.thread;
    }
};
struct WsEntry {
    void* ptr = nullptr;
    size_t bytes = 0;
    int dev = 0;
};
std::mutex g_mu;
std::unordered_map<WsKey, WsEntry, WsHash> g_ws;
// Buffers replaced by larger ones.  They are not freed when replaced: a HIP graph captured
// earlier may hold their address and replay later, and another host thread may have been handed
// the pointer and not yet queued its kernels.  mss_release_workspaces() frees them.
std::vector<std::pair<int, void*>> g_retired;
std::unordered_map<int, int> g_cus;

// Test and tuning overrides (mss_set_plan_overrides); zero = automatic plan.
std::atomic<int> g_force_generic{0};
std::atomic<int> g_generic_segments{0};
std::atomic<int64_t> g_fast_waves{0};
std::atomic<int> g_bwd_segments{0};
std::atomic<int> g_ssd_segments{0};

hipError_t device_cus(int dev, int* cus) {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_cus.find(dev);
    if (it != g_cus.end()) {
        *cus = it->second;
        return hipSuccess;
    }
    int v = 0;
    hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    g_cus[dev] = v;
    *cus = v;
    return hipSuccess;
}

// The workspace of (dev, stream) with at least `bytes`, in *out.  Returns MSS_OK, MSS_ERR_HIP, or
// MSS_ERR_UNSUPPORTED when the buffer would have to grow while `stream` is being captured into a
// graph (nothing can be allocated then: a call of at least the same size on that stream must come
// first).
int workspace(int dev, void* stream, size_t bytes, float** out) {
    std::lock_guard<std::mutex> lk(g_mu);
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    const size_t tid = hs == hipStreamPerThread ? std::hash<std::thread::id>()(std::this_thread::get_id()) : 0;
    WsEntry& w = g_ws[WsKey{dev, stream, tid}];
    if (w.bytes < bytes) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(hs, &cs) != hipSuccess) return MSS_ERR_HIP;
        if (cs != hipStreamCaptureStatusNone) return MSS_ERR_UNSUPPORTED;
        const size_t grown = bytes + bytes / 4;
        void* p = nullptr;
        if (hipMalloc(&p, grown) != hipSuccess) return MSS_ERR_HIP;
        if (w.ptr) g_retired.emplace_back(w.dev, w.ptr);
        w.ptr = p;
        w.bytes = grown;
        w.dev = dev;
    }
    *out = static_cast<float*>(w.ptr);
    return MSS_OK;
}

// ---- the scratch of mss_selective_scan_fwd_noalloc: a fixed array in device memory, one copy per
// GPU, owned by the loaded library for the life of the process.  Host code never uses the name
// `scratch` as an address (on the host it is only a stand-in for the symbol): each device's
// address comes from hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = size_t{16} << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::unordered_map<int, void*> g_scratch_ptr;

// This device's scratch address in *out (g_mu is taken here).
hipError_t scratch_of(int dev, void** out) {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_scratch_ptr.find(dev);
    if (it != g_scratch_ptr.end()) {
        *out = it->second;
        return hipSuccess;
    }
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
    *out = ptr;
    return hipSuccess;
}

// Launch timing (mss_profile_enable / mss_profile_fwd): one event triple per recorded call.
constexpr int kProfMaxCalls = 1024;
struct Prof {
    bool on = false;
    int calls = 0;                 // recorded since enabling
    std::vector<hipEvent_t> ev;    // 3 per call slot, created on demand
    std::vector<char> split;       // the call ran a carry stage
};
Prof g_prof;

int validate_fwd(const mss_tensor_t* u, const mss_tensor_t* delta, const mss_tensor_t* A,
                 const mss_tensor_t* B, const mss_tensor_t* C, const mss_tensor_t* D,
                 const mss_tensor_t* z, const mss_tensor_t* bias, const mss_tensor_t* h0,
                 const mss_tensor_t* out, const mss_tensor_t* last) {
    {
        const mss_tensor_t* const req[] = {u, delta, A, B, C, out};
        const int s = check_descs(req, {D, z, bias, h0, last});
        if (s != MSS_OK) return s;
    }
    if (u->ndim != 3 || A->ndim != 2) return MSS_ERR_SHAPE;
    const int64_t Bt = u->shape[0], Dn = u->shape[1], L = u->shape[2], N = A->shape[1];
    if (Bt < 0 || Dn < 0 || L < 0 || N < 0) return MSS_ERR_SHAPE;
    if (!shape_is(*delta, 3, Bt, Dn, L) || !shape_is(*out, 3, Bt, Dn, L)) return MSS_ERR_SHAPE;
    if (z && !shape_is(*z, 3, Bt, Dn, L)) return MSS_ERR_SHAPE;
    if (!shape_is(*A, 2, Dn, N)) return MSS_ERR_SHAPE;
    if (!shape_is(*B, 3, Bt, N, L) || !shape_is(*C, 3, Bt, N, L)) return MSS_ERR_SHAPE;
    if (D && !shape_is(*D, 1, Dn)) return MSS_ERR_SHAPE;
    if (bias && !shape_is(*bias, 1, Dn)) return MSS_ERR_SHAPE;
    if (last && !shape_is(*last, 3, Bt, Dn, N)) return MSS_ERR_SHAPE;
    if (h0 && !shape_is(*h0, 3, Bt, Dn, N)) return MSS_ERR_SHAPE;

    if (u->dtype != MSS_F32 && u->dtype != MSS_BF16) return MSS_ERR_DTYPE;
    if (delta->dtype != u->dtype || out->dtype != u->dtype || (z && z->dtype != u->dtype))
        return MSS_ERR_DTYPE;
    if (A->dtype != MSS_F32 || B->dtype != MSS_F32 || C->dtype != MSS_F32) return MSS_ERR_DTYPE;
    if ((D && D->dtype != MSS_F32) || (bias && bias->dtype != MSS_F32) || (last && last->dtype != MSS_F32) ||
        (h0 && h0->dtype != MSS_F32))
        return MSS_ERR_DTYPE;

    const mss_tensor_t* all[] = {u, delta, A, B, C, D, z, bias, h0, out, last};
    for (const mss_tensor_t* t : all) {
        if (!t) continue;
        if (!dense(*t) || !aligned(*t, elem_size(t->dtype))) return MSS_ERR_LAYOUT;
    }
    if (!aligned(*A, 16) || (last && !aligned(*last, 16)) || (h0 && !aligned(*h0, 16)))
        return MSS_ERR_LAYOUT;

    const mss_tensor_t* ins[] = {u, delta, A, B, C, D, z, bias, h0};
    for (const mss_tensor_t* t : ins) {
        if (overlap(out, t)) return MSS_ERR_ALIAS;
        if (last && overlap(last, t)) return MSS_ERR_ALIAS;
    }
    if (last && overlap(out, last)) return MSS_ERR_ALIAS;

    if (N != 16 && N != 32 && N != 64 && N != 128) return MSS_ERR_UNSUPPORTED;
    if (Bt > 65535) return MSS_ERR_UNSUPPORTED;
    return MSS_OK;
}

int validate_decode(const mss_tensor_t* state, const mss_tensor_t* x, const mss_tensor_t* dt,
                    const mss_tensor_t* A, const mss_tensor_t* B, const mss_tensor_t* C,
                    const mss_tensor_t* D, const mss_tensor_t* z, const mss_tensor_t* bias,
                    const mss_tensor_t* out) {
    {
        const mss_tensor_t* const req[] = {state, x, dt, A, B, C, out};
        const int s = check_descs(req, {D, z, bias});
        if (s != MSS_OK) return s;
    }
    if (state->ndim != 3) return MSS_ERR_SHAPE;
    const int64_t Bt = state->shape[0], Dn = state->shape[1], N = state->shape[2];
    if (Bt < 0 || Dn < 0 || N < 0) return MSS_ERR_SHAPE;
    if (!shape_is(*x, 2, Bt, Dn) || !shape_is(*dt, 2, Bt, Dn) || !shape_is(*out, 2, Bt, Dn))
        return MSS_ERR_SHAPE;
    if (z && !shape_is(*z, 2, Bt, Dn)) return MSS_ERR_SHAPE;
    if (!shape_is(*A, 2, Dn, N) || !shape_is(*B, 2, Bt, N) || !shape_is(*C, 2, Bt, N))
        return MSS_ERR_SHAPE;
    if (D && !shape_is(*D, 1, Dn)) return MSS_ERR_SHAPE;
    if (bias && !shape_is(*bias, 1, Dn)) return MSS_ERR_SHAPE;

    if (x->dtype != MSS_F32 && x->dtype != MSS_BF16) return MSS_ERR_DTYPE;
    if (dt->dtype != x->dtype || out->dtype != x->dtype || (z && z->dtype != x->dtype))
        return MSS_ERR_DTYPE;
    if (state->dtype != MSS_F32 || A->dtype != MSS_F32 || B->dtype != MSS_F32 || C->dtype != MSS_F32)
        return MSS_ERR_DTYPE;
    if ((D && D->dtype != MSS_F32) || (bias && bias->dtype != MSS_F32)) return MSS_ERR_DTYPE;

    const mss_tensor_t* all[] = {state, x, dt, A, B, C, D, z, bias, out};
    for (const mss_tensor_t* t : all) {
        if (!t) continue;
        if (!dense(*t) || !aligned(*t, elem_size(t->dtype))) return MSS_ERR_LAYOUT;
    }
    if (!aligned(*state, 16) || !aligned(*A, 16) || !aligned(*B, 16) || !aligned(*C, 16))
        return MSS_ERR_LAYOUT;

    const mss_tensor_t* ins[] = {x, dt, A, B, C, D, z, bias};
    for (const mss_tensor_t* t : ins) {
        if (overlap(out, t) || overlap(state, t)) return MSS_ERR_ALIAS;
    }
    if (overlap(out, state)) return MSS_ERR_ALIAS;

    if (N != 16 && N != 32 && N != 64 && N != 128) return MSS_ERR_UNSUPPORTED;
    return MSS_OK;
}

int validate_bwd(const mss_tensor_t* u, const mss_tensor_t* delta, const mss_tensor_t* A,
                 const mss_tensor_t* B, const mss_tensor_t* C, const mss_tensor_t* D,
                 const mss_tensor_t* z, const mss_tensor_t* bias, const mss_tensor_t* dout,
                 const mss_tensor_t* du, const mss_tensor_t* ddelta, const mss_tensor_t* dA,
                 const mss_tensor_t* dB, const mss_tensor_t* dC, const mss_tensor_t* dD,
                 const mss_tensor_t* dz, const mss_tensor_t* dbias) {
    {
        const mss_tensor_t* const req[] = {u, delta, A, B, C, dout, du, ddelta, dA, dB, dC};
        const int s = check_descs(req, {D, z, bias, dD, dz, dbias});
        if (s != MSS_OK) return s;
    }
    if (u->ndim != 3 || A->ndim != 2) return MSS_ERR_SHAPE;
    const int64_t Bt = u->shape[0], Dn = u->shape[1], L = u->shape[2], N = A->shape[1];
    if (Bt < 0 || Dn < 0 || L < 0 || N < 0) return MSS_ERR_SHAPE;
    for (const mss_tensor_t* t : {delta, dout, du, ddelta})
        if (!shape_is(*t, 3, Bt, Dn, L)) return MSS_ERR_SHAPE;
    if (z && !shape_is(*z, 3, Bt, Dn, L)) return MSS_ERR_SHAPE;
    if (dz && (!z || !shape_is(*dz, 3, Bt, Dn, L))) return MSS_ERR_SHAPE;  // no gate, no dz
    if (!shape_is(*A, 2, Dn, N) || !shape_is(*dA, 2, Dn, N)) return MSS_ERR_SHAPE;
    for (const mss_tensor_t* t : {B, C, dB, dC})
        if (!shape_is(*t, 3, Bt, N, L)) return MSS_ERR_SHAPE;
    for (const mss_tensor_t* t : {D, bias, dD, dbias})
        if (t && !shape_is(*t, 1, Dn)) return MSS_ERR_SHAPE;

    if (u->dtype != MSS_F32 && u->dtype != MSS_BF16) return MSS_ERR_DTYPE;
    for (const mss_tensor_t* t : {delta, dout, du, ddelta, z, dz})
        if (t && t->dtype != u->dtype) return MSS_ERR_DTYPE;
    for (const mss_tensor_t* t : {A, B, C, D, bias, dA, dB, dC, dD, dbias})
        if (t && t->dtype != MSS_F32) return MSS_ERR_DTYPE;

    const mss_tensor_t* all[] = {u, delta, A, B, C, D, z, bias, dout, du, ddelta, dA, dB, dC, dD, dz, dbias};
    for (const mss_tensor_t* t : all) {
        if (!t) continue;
        if (!dense(*t) || !aligned(*t, elem_size(t->dtype))) return MSS_ERR_LAYOUT;
    }
    if (!aligned(*A, 16)) return MSS_ERR_LAYOUT;

    const mss_tensor_t* ins[] = {u, delta, A, B, C, D, z, bias, dout};
    const mss_tensor_t* outs[] = {du, ddelta, dA, dB, dC, dD, dz, dbias};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const mss_tensor_t* t : ins)
            if (overlap(outs[i], t)) return MSS_ERR_ALIAS;
        for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
            if (overlap(outs[i], outs[j])) return MSS_ERR_ALIAS;
    }

    if (N != kN) return MSS_ERR_UNSUPPORTED;
    if (Bt > 65535) return MSS_ERR_UNSUPPORTED;
    return MSS_OK;
}

constexpr int kMaxConvK = 4;

int validate_conv_fwd(const mss_tensor_t* x, const mss_tensor_t* w, const mss_tensor_t* bias,
                      const mss_tensor_t* st_in, const mss_tensor_t* out, const mss_tensor_t* st_out) {
    {
        const mss_tensor_t* const req[] = {x, w, out};
        const int s = check_descs(req, {bias, st_in, st_out});
        if (s != MSS_OK) return s;
    }
    if (x->ndim != 3 || w->ndim != 2) return MSS_ERR_SHAPE;
    const int64_t Bt = x->shape[0], Dn = x->shape[1], L = x->shape[2], K = w->shape[1];
    if (Bt < 0 || Dn < 0 || L < 0 || K < 1) return MSS_ERR_SHAPE;
    if (!shape_is(*w, 2, Dn, K) || !shape_is(*out, 3, Bt, Dn, L)) return MSS_ERR_SHAPE;
    if (bias && !shape_is(*bias, 1, Dn)) return MSS_ERR_SHAPE;
    for (const mss_tensor_t* t : {st_in, st_out})
        if (t && !shape_is(*t, 3, Bt, Dn, K - 1)) return MSS_ERR_SHAPE;
    if (x->dtype != MSS_F32 && x->dtype != MSS_BF16) return MSS_ERR_DTYPE;
    for (const mss_tensor_t* t : {out, st_in, st_out})
        if (t && t->dtype != x->dtype) return MSS_ERR_DTYPE;
    if (w->dtype != MSS_F32 || (bias && bias->dtype != MSS_F32)) return MSS_ERR_DTYPE;
    for (const mss_tensor_t* t : {x, w, bias, st_in, out, st_out}) {
        if (!t) continue;
        if (!dense(*t) || !aligned(*t, elem_size(t->dtype))) return MSS_ERR_LAYOUT;
    }
    for (const mss_tensor_t* t : {x, w, bias, st_in}) {
        if (overlap(out, t)) return MSS_ERR_ALIAS;
        if (st_out && overlap(st_out, t)) return MSS_ERR_ALIAS;
    }
    if (st_out && overlap(st_out, out)) return MSS_ERR_ALIAS;
    if (K > kMaxConvK) return MSS_ERR_UNSUPPORTED;
    return MSS_OK;
}

int validate_conv_update(const mss_tensor_t* st, const mss_tensor_t* x, const mss_tensor_t* w,
                         const mss_tensor_t* bias, const mss_tensor_t* out) {
    {
        const mss_tensor_t* const req[] = {st, x, w, out};
        const int s = check_descs(req, {bias});
        if (s != MSS_OK) return s;
    }
    if (x->ndim != 2 || w->ndim != 2) return MSS_ERR_SHAPE;
    const int64_t Bt = x->shape[0], Dn = x->shape[1], K = w->shape[1];
    if (Bt < 0 || Dn < 0 || K < 1) return MSS_ERR_SHAPE;
    if (!shape_is(*w, 2, Dn, K) || !shape_is(*out, 2, Bt, Dn) || !shape_is(*st, 3, Bt, Dn, K - 1))
        return MSS_ERR_SHAPE;
    if (bias && !shape_is(*bias, 1, Dn)) return MSS_ERR_SHAPE;
    if (x->dtype != MSS_F32 && x->dtype != MSS_BF16) return MSS_ERR_DTYPE;
    if (st->dtype != x->dtype || out->dtype != x->dtype) return MSS_ERR_DTYPE;
    if (w->dtype != MSS_F32 || (bias && bias->dtype != MSS_F32)) return MSS_ERR_DTYPE;
    for (const mss_tensor_t* t : {st, x, w, bias, out}) {
        if (!t) continue;
        if (!dense(*t) || !aligned(*t, elem_size(t->dtype))) return MSS_ERR_LAYOUT;
    }
    for (const mss_tensor_t* t : {x, w, bias}) {
        if (overlap(out, t) || overlap(st, t)) return MSS_ERR_ALIAS;
    }
    if (overlap(out, st)) return MSS_ERR_ALIAS;
    if (K > kMaxConvK) return MSS_ERR_UNSUPPORTED;
    return MSS_OK;
}

}  // namespace

extern "C" {

int mss_version(void) { return MSS_VERSION; }

const char* mss_status_string(int status) {
    switch (status) {
        case MSS_OK: return "MSS_OK";
        case MSS_ERR_NULL_ARG: return "MSS_ERR_NULL_ARG";
        case MSS_ERR_SHAPE: return "MSS_ERR_SHAPE";
        case MSS_ERR_DTYPE: return "MSS_ERR_DTYPE";
        case MSS_ERR_LAYOUT: return "MSS_ERR_LAYOUT";
        case MSS_ERR_ALIAS: return "MSS_ERR_ALIAS";
        case MSS_ERR_UNSUPPORTED: return "MSS_ERR_UNSUPPORTED";
        case MSS_ERR_HIP: return "MSS_ERR_HIP";
        default: return "MSS_ERR_UNKNOWN";
    }
}

int mss_selective_scan_fwd(const mss_tensor_t* u, const mss_tensor_t* delta, const mss_tensor_t* A,
                           const mss_tensor_t* B, const mss_tensor_t* C, const mss_tensor_t* D,
                           const mss_tensor_t* z, const mss_tensor_t* delta_bias, int softplus_flag,
                           const mss_tensor_t* out, const mss_tensor_t* last_state, void* stream) {
    return mss_selective_scan_fwd_with_state(u, delta, A, B, C, D, z, delta_bias, nullptr, softplus_flag,
                                             out, last_state, stream);
}

int mss_selective_scan_fwd_with_state(const mss_tensor_t* u, const mss_tensor_t* delta,
                                      const mss_tensor_t* A, const mss_tensor_t* B,
                                      const mss_tensor_t* C, const mss_tensor_t* D,
                                      const mss_tensor_t* z, const mss_tensor_t* delta_bias,
                                      const mss_tensor_t* initial_state, int softplus_flag,
                                      const mss_tensor_t* out, const mss_tensor_t* last_state,
                                      void* stream) {
    return mss_selective_scan_fwd_varlen(u, delta, A, B, C, D, z, delta_bias, initial_state, nullptr,
                                         softplus_flag, out, last_state, stream);
}

int mss_selective_scan_fwd_varlen(const mss_tensor_t* u, const mss_tensor_t* delta,
                                  const mss_tensor_t* A, const mss_tensor_t* B,
                                  const mss_tensor_t* C, const mss_tensor_t* D,
                                  const mss_tensor_t* z, const mss_tensor_t* delta_bias,
                                  const mss_tensor_t* initial_state, const mss_tensor_t* seq_lens,
                                  int softplus_flag, const mss_tensor_t* out,
                                  const mss_tensor_t* last_state, void* stream) {
    return mss_selective_scan_fwd_save(u, delta, A, B, C, D, z, delta_bias, initial_state, seq_lens,
                                       softplus_flag, out, last_state, nullptr, stream);
}

namespace {
// The states saved for the backward: (ceil(L / 8), d_state / 4, batch * d_inner * 4) f32, planes
// of float4 (states 4q..4q+3 of each row).
int check_saved(const mss_tensor_t* saved, const mss_tensor_t* u, int64_t N) {
    const int st = check_desc(saved, true);
    if (st != MSS_OK) return st;
    const int64_t Bt = u->shape[0], Dn = u->shape[1], L = u->shape[2];
    if (!shape_is(*saved, 3, (L + 7) / 8, N / 4, Bt * Dn * 4)) return MSS_ERR_SHAPE;
    if (saved->dtype != MSS_F32) return MSS_ERR_DTYPE;
    if (!dense(*saved) || !aligned(*saved, 16)) return MSS_ERR_LAYOUT;
    return MSS_OK;
}
}  // namespace

int mss_selective_scan_fwd_save(const mss_tensor_t* u, const mss_tensor_t* delta,
                                const mss_tensor_t* A, const mss_tensor_t* B,
                                const mss_tensor_t* C, const mss_tensor_t* D,
                                const mss_tensor_t* z, const mss_tensor_t* delta_bias,
                                const mss_tensor_t* initial_state, const mss_tensor_t* seq_lens,
                                int softplus_flag, const mss_tensor_t* out,
                                const mss_tensor_t* last_state, const mss_tensor_t* saved_states,
                                void* stream) {
    try {
        int st = validate_fwd(u, delta, A, B, C, D, z, delta_bias, initial_state, out, last_state);
        if (st != MSS_OK) return st;
        if (saved_states) {
            if (A->shape[1] != kN) return MSS_ERR_UNSUPPORTED;  // the backward that reads them is d_state 16
            st = check_saved(saved_states, u, A->shape[1]);
            if (st != MSS_OK) return st;
            for (const mss_tensor_t* t : {u, delta, A, B, C, D, z, delta_bias, initial_state, seq_lens, out,
                                          last_state})
                if (t && overlap(saved_states, t)) return MSS_ERR_ALIAS;
        }
        if (seq_lens) {
            st = check_desc(seq_lens, false);
            if (st != MSS_OK) return st;
            if (!shape_is(*seq_lens, 1, u->shape[0])) return MSS_ERR_SHAPE;
            if (seq_lens->dtype != MSS_I32) return MSS_ERR_DTYPE;
            if (!dense(*seq_lens) || !aligned(*seq_lens, 4)) return MSS_ERR_LAYOUT;
            if (overlap(out, seq_lens) || (last_state && overlap(last_state, seq_lens))) return MSS_ERR_ALIAS;
        }
        mss::ScanLaunch a;
        a.u = u->data; a.delta = delta->data; a.z = z ? z->data : nullptr;
        a.A = static_cast<const float*>(A->data);
        a.B = static_cast<const float*>(B->data);
        a.C = static_cast<const float*>(C->data);
        a.D = D ? static_cast<const float*>(D->data) : nullptr;
        a.bias = delta_bias ? static_cast<const float*>(delta_bias->data) : nullptr;
        a.out = out->data;
        a.last_state = last_state ? static_cast<float*>(last_state->data) : nullptr;
        a.h0 = initial_state ? static_cast<const float*>(initial_state->data) : nullptr;
        a.lens = (seq_lens && numel(*seq_lens) > 0) ? static_cast<const int32_t*>(seq_lens->data) : nullptr;
        a.saved = (saved_states && numel(*saved_states) > 0) ? static_cast<float*>(saved_states->data) : nullptr;
        a.Bt = u->shape[0]; a.Dn = u->shape[1]; a.L = u->shape[2]; a.N = static_cast<int>(A->shape[1]);
        a.softplus = softplus_flag ? 1 : 0;
        a.bf16 = u->dtype == MSS_BF16;
        const size_t es = elem_size(u->dtype);
        a.vec_ok = (a.L * static_cast<int64_t>(es)) % 16 == 0 && aligned(*u, 16) &&
                   aligned(*delta, 16) && aligned(*out, 16) && (!z || aligned(*z, 16)) &&
                   aligned(*B, 16) && aligned(*C, 16);
        if (a.Bt * a.Dn == 0) return MSS_OK;

        hipStream_t s = static_cast<hipStream_t>(stream);
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess) return MSS_ERR_HIP;
        if (device_cus(dev, &cus) != hipSuccess) return MSS_ERR_HIP;
        // the fast path takes every length at d_state 16 (rows that are not whole 16-byte vectors
        // run its element-aligned variant); the generic kernels run for L = 0, for d_state 32, 64
        // and 128, and when a test forces them
        bool fast = a.L > 0 && a.N == kN && (a.saved || g_force_generic.load() == 0);
        mss::ScanPlan plan;
        if (fast) {
            plan = mss::plan_fast(a, cus, g_fast_waves.load());
            // 2^32 (64-channel group, 16- or 32-step tile) pairs and more: the generic kernels
            // (only the state-saving variant has no generic form)
            if (!plan.fits) {
                if (a.saved) return MSS_ERR_UNSUPPORTED;
                fast = false;
            }
        }
        if (!fast) {
            plan = mss::plan_scan(a, cus, mss::generic_tile(), g_generic_segments.load());
            plan.workspace_bytes = mss::generic_workspace_bytes(a, plan.segments);
        }
        float* ws = nullptr;
        if (plan.workspace_bytes > 0) {
            const int wst = workspace(dev, stream, plan.workspace_bytes, &ws);
            if (wst != MSS_OK) return wst;
        }
        std::unique_lock<std::mutex> plk(g_mu, std::defer_lock);
        int slot = -1;
        if (g_prof.on) {
            plk.lock();
            if (g_prof.calls < kProfMaxCalls) {
                slot = g_prof.calls;
                if (static_cast<int>(g_prof.split.size()) <= slot) {
                    for (int k = 0; k < 3; ++k) {
                        hipEvent_t ev = nullptr;
                        if (hipEventCreate(&ev) != hipSuccess) return MSS_ERR_HIP;
                        g_prof.ev.push_back(ev);
                    }
                    g_prof.split.push_back(0);
                }
                for (int k = 0; k < 3; ++k) a.ev[k] = g_prof.ev[3 * slot + k];
                g_prof.split[slot] = plan.segments > 1;
            }
        }
        const hipError_t e = fast ? mss::launch_scan_fast(a, plan, ws, s) : mss::launch_scan_fwd(a, plan, ws, s);
        if (slot >= 0 && e == hipSuccess) g_prof.calls = slot + 1;
        return e == hipSuccess ? MSS_OK : MSS_ERR_HIP;
    } catch (...) {
        return MSS_ERR_HIP;
    }
}

int mss_selective_scan_fwd_noalloc(const mss_tensor_t* u, const mss_tensor_t* delta, const mss_tensor_t* A,
                                   const mss_tensor_t* B, const mss_tensor_t* C, const mss_tensor_t* D,
                                   const mss_tensor_t* z, const mss_tensor_t* delta_bias, int softplus_flag,
                                   const mss_tensor_t* out, const mss_tensor_t* last_state, void* stream) {
    try {
        const int st = validate_fwd(u, delta, A, B, C, D, z, delta_bias, nullptr, out, last_state);
        if (st != MSS_OK) return st;
        if (A->shape[1] != kN) return MSS_ERR_UNSUPPORTED;  // the fast kernels only: d_state 16
        // a forced wavefront count whose aggregates cannot fit: refused before any HIP call
        const int64_t forced = g_fast_waves.load();
        const size_t slot_bytes = (kN + 1) * 64 * sizeof(float);
        if (forced > 0 && static_cast<size_t>(forced) > kScratchBytes / slot_bytes) return MSS_ERR_UNSUPPORTED;
        mss::ScanLaunch a;
        a.u = u->data; a.delta = delta->data; a.z = z ? z->data : nullptr;
        a.A = static_cast<const float*>(A->data);
        a.B = static_cast<const float*>(B->data);
        a.C = static_cast<const float*>(C->data);
        a.D = D ? static_cast<const float*>(D->data) : nullptr;
        a.bias = delta_bias ? static_cast<const float*>(delta_bias->data) : nullptr;
        a.out = out->data;
        a.last_state = last_state ? static_cast<float*>(last_state->data) : nullptr;
        a.h0 = nullptr;
        a.lens = nullptr;
        a.saved = nullptr;
        a.Bt = u->shape[0]; a.Dn = u->shape[1]; a.L = u->shape[2];
        a.softplus = softplus_flag ? 1 : 0;
        a.bf16 = u->dtype == MSS_BF16;
        const size_t es = elem_size(u->dtype);
        a.vec_ok = (a.L * static_cast<int64_t>(es)) % 16 == 0 && aligned(*u, 16) &&
                   aligned(*delta, 16) && aligned(*out, 16) && (!z || aligned(*z, 16)) &&
                   aligned(*B, 16) && aligned(*C, 16);
        if (a.Bt * a.Dn == 0) return MSS_OK;

        hipStream_t s = static_cast<hipStream_t>(stream);
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess) return MSS_ERR_HIP;
        if (device_cus(dev, &cus) != hipSuccess) return MSS_ERR_HIP;
        void* base = nullptr;
        if (scratch_of(dev, &base) != hipSuccess) return MSS_ERR_HIP;
        if (a.L == 0) {  // no scan steps: last_state <- zeros (no scratch)
            mss::ScanPlan none{};
            return mss::launch_scan_fwd(a, none, nullptr, s) == hipSuccess ? MSS_OK : MSS_ERR_HIP;
        }
        // the fast kernels only (the generic ones need scratch in proportion to the rows); the
        // automatic wavefront count is capped so that its aggregates fit the scratch
        mss::ScanPlan plan = mss::plan_fast(a, cus, forced);
        const int64_t cap = static_cast<int64_t>(kScratchBytes / slot_bytes);
        if (forced == 0 && plan.waves > cap) plan = mss::plan_fast(a, cus, cap);
        if (!plan.fits || plan.workspace_bytes > kScratchBytes) return MSS_ERR_UNSUPPORTED;
        float* ws = plan.workspace_bytes > 0 ? static_cast<float*>(base) : nullptr;
        return mss::launch_scan_fast(a, plan, ws, s) == hipSuccess ? MSS_OK : MSS_ERR_HIP;
    } catch (...) {
        return MSS_ERR_HIP;
    }
}

int mss_selective_scan_bwd(const mss_tensor_t* u, const mss_tensor_t* delta, const mss_tensor_t* A,
                           const mss_tensor_t* B, const mss_tensor_t* C, const mss_tensor_t* D,
                           const mss_tensor_t* z, const mss_tensor_t* delta_bias, int softplus_flag,
                           const mss_tensor_t* dout, const mss_tensor_t* du, const mss_tensor_t* ddelta,
                           const mss_tensor_t* dA, const mss_tensor_t* dB, const mss_tensor_t* dC,
                           const mss_tensor_t* dD, const mss_tensor_t* dz,
                           const mss_tensor_t* ddelta_bias, void* stream) {
    return mss_selective_scan_bwd_varlen(u, delta, A, B, C, D, z, delta_bias, nullptr, nullptr, softplus_flag,
                                         dout, nullptr, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, nullptr,
                                         stream);
}

namespace {
int bwd_impl(const mss_tensor_t* u, const mss_tensor_t* delta, const mss_tensor_t* A, const mss_tensor_t* B,
             const mss_tensor_t* C, const mss_tensor_t* D, const mss_tensor_t* z, const mss_tensor_t* delta_bias,
             const mss_tensor_t* initial_state, const mss_tensor_t* seq_lens, const mss_tensor_t* saved,
             int softplus_flag, const mss_tensor_t* dout, const mss_tensor_t* dlast_state, const mss_tensor_t* du,
             const mss_tensor_t* ddelta, const mss_tensor_t* dA, const mss_tensor_t* dB, const mss_tensor_t* dC,
             const mss_tensor_t* dD, const mss_tensor_t* dz, const mss_tensor_t* ddelta_bias,
             const mss_tensor_t* dinitial_state, void* stream) {
    try {
        int st = validate_bwd(u, delta, A, B, C, D, z, delta_bias, dout, du, ddelta, dA, dB, dC, dD,
                              dz, ddelta_bias);
        if (st != MSS_OK) return st;
        if (saved) {
            st = check_saved(saved, u, A->shape[1]);
            if (st != MSS_OK) return st;
            for (const mss_tensor_t* o : {du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dinitial_state})
                if (o && overlap(o, saved)) return MSS_ERR_ALIAS;
        }
        {
            // the state tensors: (Bt, Dn, N) f32, 16-byte aligned; the lengths: (Bt,) i32
            const int64_t Bt = u->shape[0], Dn = u->shape[1], N = A->shape[1];
            for (const mss_tensor_t* t : {initial_state, dlast_state, dinitial_state, seq_lens}) {
                st = check_desc(t, false);
                if (st != MSS_OK) return st;
            }
            for (const mss_tensor_t* t : {initial_state, dlast_state, dinitial_state}) {
                if (!t) continue;
                if (!shape_is(*t, 3, Bt, Dn, N)) return MSS_ERR_SHAPE;
                if (t->dtype != MSS_F32) return MSS_ERR_DTYPE;
                if (!dense(*t) || !aligned(*t, 16)) return MSS_ERR_LAYOUT;
            }
            if (seq_lens) {
                if (!shape_is(*seq_lens, 1, Bt)) return MSS_ERR_SHAPE;
                if (seq_lens->dtype != MSS_I32) return MSS_ERR_DTYPE;
                if (!dense(*seq_lens) || !aligned(*seq_lens, 4)) return MSS_ERR_LAYOUT;
            }
            const mss_tensor_t* outs[] = {du, ddelta, dA, dB, dC, dD, dz, ddelta_bias};
            for (const mss_tensor_t* o : outs)
                for (const mss_tensor_t* t : {initial_state, dlast_state, seq_lens, dinitial_state})
                    if (o && overlap(o, t)) return MSS_ERR_ALIAS;
            if (dinitial_state)
                for (const mss_tensor_t* t : {u, delta, A, B, C, D, z, delta_bias, dout, initial_state,
                                              dlast_state, seq_lens})
                    if (overlap(dinitial_state, t)) return MSS_ERR_ALIAS;
        }
        mss::BwdLaunch a;
        a.u = u->data; a.delta = delta->data; a.z = z ? z->data : nullptr; a.dout = dout->data;
        a.A = static_cast<const float*>(A->data);
        a.B = static_cast<const float*>(B->data);
        a.C = static_cast<const float*>(C->data);
        a.D = D ? static_cast<const float*>(D->data) : nullptr;
        a.bias = delta_bias ? static_cast<const float*>(delta_bias->data) : nullptr;
        a.du = du->data; a.ddelta = ddelta->data; a.dz = dz ? dz->data : nullptr;
        a.dA = static_cast<float*>(dA->data);
        a.dB = static_cast<float*>(dB->data);
        a.dC = static_cast<float*>(dC->data);
        a.dD = dD ? static_cast<float*>(dD->data) : nullptr;
        a.dbias = ddelta_bias ? static_cast<float*>(ddelta_bias->data) : nullptr;
        a.h0 = initial_state ? static_cast<const float*>(initial_state->data) : nullptr;
        a.lens = (seq_lens && numel(*seq_lens) > 0) ? static_cast<const int32_t*>(seq_lens->data) : nullptr;
        a.dlast = dlast_state ? static_cast<const float*>(dlast_state->data) : nullptr;
        a.dh0 = dinitial_state ? static_cast<float*>(dinitial_state->data) : nullptr;
        a.saved = (saved && numel(*saved) > 0) ? static_cast<const float*>(saved->data) : nullptr;
        a.Bt = u->shape[0]; a.Dn = u->shape[1]; a.L = u->shape[2];
        a.softplus = softplus_flag ? 1 : 0;
        a.bf16 = u->dtype == MSS_BF16;
        const size_t es = elem_size(u->dtype);
        a.vec_ok = (a.L * static_cast<int64_t>(es)) % 16 == 0 && aligned(*u, 16) && aligned(*delta, 16) &&
                   aligned(*dout, 16) && aligned(*du, 16) && aligned(*ddelta, 16) && (!z || aligned(*z, 16)) &&
                   (!dz || aligned(*dz, 16)) && aligned(*B, 16) && aligned(*C, 16);
        const int64_t elems = a.Dn * kN + a.Bt * kN * a.L + a.Dn + (a.dh0 ? a.Bt * a.Dn * kN : 0);
        if (elems == 0) return MSS_OK;  // nothing to write

        hipStream_t s = static_cast<hipStream_t>(stream);
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess) return MSS_ERR_HIP;
        if (device_cus(dev, &cus) != hipSuccess) return MSS_ERR_HIP;
        const int segments = mss::plan_bwd_segments(a, cus, g_bwd_segments.load());
        const size_t bytes = mss::bwd_workspace_bytes(a, segments);
        float* ws = nullptr;
        if (bytes > 0) {
            const int wst = workspace(dev, stream, bytes, &ws);
            if (wst != MSS_OK) return wst;
        }
        return mss::launch_scan_bwd(a, segments, ws, s) == hipSuccess ? MSS_OK : MSS_ERR_HIP;
    } catch (...) {
        return MSS_ERR_HIP;
    }
}
}  // namespace

int mss_selective_scan_bwd_varlen(const mss_tensor_t* u, const mss_tensor_t* delta, const mss_tensor_t* A,
                                  const mss_tensor_t* B, const mss_tensor_t* C, const mss_tensor_t* D,
                                  const mss_tensor_t* z, const mss_tensor_t* delta_bias,
                                  const mss_tensor_t* initial_state, const mss_tensor_t* seq_lens,
                                  int softplus_flag, const mss_tensor_t* dout,
                                  const mss_tensor_t* dlast_state, const mss_tensor_t* du,
                                  const mss_tensor_t* ddelta, const mss_tensor_t* dA, const mss_tensor_t* dB,
                                  const mss_tensor_t* dC, const mss_tensor_t* dD, const mss_tensor_t* dz,
                                  const mss_tensor_t* ddelta_bias, const mss_tensor_t* dinitial_state,
                                  void* stream) {
    return bwd_impl(u, delta, A, B, C, D, z, delta_bias, initial_state, seq_lens, nullptr, softplus_flag, dout,
                    dlast_state, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dinitial_state, stream);
}

int mss_selective_scan_bwd_saved(const mss_tensor_t* u, const mss_tensor_t* delta, const mss_tensor_t* A,
                                 const mss_tensor_t* B, const mss_tensor_t* C, const mss_tensor_t* D,
                                 const mss_tensor_t* z, const mss_tensor_t* delta_bias,
                                 const mss_tensor_t* seq_lens, int softplus_flag,
                                 const mss_tensor_t* saved_states, const mss_tensor_t* dout,
                                 const mss_tensor_t* dlast_state, const mss_tensor_t* du,
                                 const mss_tensor_t* ddelta, const mss_tensor_t* dA, const mss_tensor_t* dB,
                                 const mss_tensor_t* dC, const mss_tensor_t* dD, const mss_tensor_t* dz,
                                 const mss_tensor_t* ddelta_bias, const mss_tensor_t* dinitial_state,
                                 void* stream) {
    if (!saved_states) return MSS_ERR_NULL_ARG;
    return bwd_impl(u, delta, A, B, C, D, z, delta_bias, nullptr, seq_lens, saved_states, softplus_flag, dout,
                    dlast_state, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dinitial_state, stream);
}

int mss_causal_conv1d_fwd(const mss_tensor_t* x, const mss_tensor_t* weight, const mss_tensor_t* bias,
                          const mss_tensor_t* initial_state, int silu_flag, const mss_tensor_t* out,
                          const mss_tensor_t* final_state, void* stream) {
    try {
        const int st = validate_conv_fwd(x, weight, bias, initial_state, out, final_state);
        if (st != MSS_OK) return st;
        mss::ConvLaunch a;
        a.x = x->data;
        a.w = static_cast<const float*>(weight->data);
        a.bias = bias ? static_cast<const float*>(bias->data) : nullptr;
        a.state_in = (initial_state && numel(*initial_state) > 0) ? initial_state->data : nullptr;
        a.out = out->data;
        a.state_out = (final_state && numel(*final_state) > 0) ? final_state->data : nullptr;
        a.Dn = x->shape[1]; a.L = x->shape[2]; a.R = x->shape[0] * x->shape[1];
        a.K = static_cast<int>(weight->shape[1]);
        a.silu = silu_flag != 0;
        a.bf16 = x->dtype == MSS_BF16;
        a.vec_ok = (a.L * static_cast<int64_t>(elem_size(x->dtype))) % 16 == 0 && aligned(*x, 16) &&
                   aligned(*out, 16);
        if (a.R == 0) return MSS_OK;
        return mss::launch_conv1d_fwd(a, static_cast<hipStream_t>(stream)) == hipSuccess ? MSS_OK : MSS_ERR_HIP;
    } catch (...) {
        return MSS_ERR_HIP;
    }
}

int mss_causal_conv1d_update(const mss_tensor_t* state, const mss_tensor_t* x, const mss_tensor_t* weight,
                             const mss_tensor_t* bias, int silu_flag, const mss_tensor_t* out, void* stream) {
    try {
        const int st = validate_conv_update(state, x, weight, bias, out);
        if (st != MSS_OK) return st;
        mss::ConvUpdateLaunch a;
        a.state = state->data;
        a.x = x->data;
        a.w = static_cast<const float*>(weight->data);
        a.bias = bias ? static_cast<const float*>(bias->data) : nullptr;
        a.out = out->data;
        a.Dn = x->shape[1]; a.R = x->shape[0] * x->shape[1];
        a.K = static_cast<int>(weight->shape[1]);
        a.silu = silu_flag != 0;
        a.bf16 = x->dtype == MSS_BF16;
        if (a.R == 0) return MSS_OK;
        return mss::launch_conv1d_update(a, static_cast<hipStream_t>(stream)) == hipSuccess ? MSS_OK : MSS_ERR_HIP;
    } catch (...) {
        return MSS_ERR_HIP;
    }
}

int mss_profile_enable(int on) {
    try {
        std::lock_guard<std::mutex> lk(g_mu);
        g_prof.on = on != 0;
        if (on) g_prof.calls = 0;
        return MSS_OK;
    } catch (...) {
        return MSS_ERR_HIP;
    }
}

int mss_profile_fwd(int* calls, double* carry_ms, double* main_ms) {
    if (!calls || !carry_ms || !main_ms) return MSS_ERR_NULL_ARG;
    try {
        std::lock_guard<std::mutex> lk(g_mu);
        double c = 0.0, m = 0.0;
        for (int i = 0; i < g_prof.calls; ++i) {
            hipEvent_t* e = &g_prof.ev[3 * i];
            if (hipEventSynchronize(e[2]) != hipSuccess) return MSS_ERR_HIP;
            float ci = 0.0f, mi = 0.0f;
            if (hipEventElapsedTime(&ci, e[0], e[1]) != hipSuccess) return MSS_ERR_HIP;
            if (hipEventElapsedTime(&mi, e[1], e[2]) != hipSuccess) return MSS_ERR_HIP;
            c += g_prof.split[i] ? ci : 0.0f;
            m += mi;
        }
        *calls = g_prof.calls;
        *carry_ms = c;
        *main_ms = m;
        return MSS_OK;
    } catch (...) {
        return MSS_ERR_HIP;
    }
}

int mss_ssd_scan_fwd(const mss_tensor_t* x, const mss_tensor_t* dt, const mss_tensor_t* A,
                     const mss_tensor_t* B, const mss_tensor_t* C, const mss_tensor_t* D,
                     const mss_tensor_t* z, const mss_tensor_t* dt_bias, int softplus_flag,
                     const mss_tensor_t* out, const mss_tensor_t* last_state, void* stream) {
    try {
        {
            const mss_tensor_t* const req[] = {x, dt, A, B, C, out};
            const int s = check_descs(req, {D, z, dt_bias, last_state});
            if (s != MSS_OK) return s;
        }
        if (x->ndim != 4 || B->ndim != 4) return MSS_ERR_SHAPE;
        const int64_t Bt = x->shape[0], L = x->shape[1], H = x->shape[2], P = x->shape[3];
        const int64_t G = B->shape[2], N = B->shape[3];
        if (!shape_is(*dt, 3, Bt, L, H) || !shape_is(*A, 1, H) || !shape_is(*out, 4, Bt, L, H, P)) return MSS_ERR_SHAPE;
        if (!shape_is(*B, 4, Bt, L, G, N) || !shape_is(*C, 4, Bt, L, G, N)) return MSS_ERR_SHAPE;
        if (z && !shape_is(*z, 4, Bt, L, H, P)) return MSS_ERR_SHAPE;
        if ((D && !shape_is(*D, 1, H)) || (dt_bias && !shape_is(*dt_bias, 1, H))) return MSS_ERR_SHAPE;
        if (last_state && !shape_is(*last_state, 4, Bt, H, P, N)) return MSS_ERR_SHAPE;
        if (G < 1 || H % G != 0) return MSS_ERR_SHAPE;  // heads come in whole blocks per group

        if (x->dtype != MSS_BF16 && x->dtype != MSS_F32) return MSS_ERR_DTYPE;
        for (const mss_tensor_t* t : {dt, B, C, out, z})
            if (t && t->dtype != x->dtype) return MSS_ERR_DTYPE;
        for (const mss_tensor_t* t : {A, D, dt_bias, last_state})
            if (t && t->dtype != MSS_F32) return MSS_ERR_DTYPE;
        for (const mss_tensor_t* t : {x, dt, A, B, C, D, z, dt_bias, out, last_state}) {
            if (!t) continue;
            if (!dense(*t) || !aligned(*t, elem_size(t->dtype))) return MSS_ERR_LAYOUT;
        }
        for (const mss_tensor_t* t : {x, B, C, z, out})  // 16-byte vector accesses
            if (t && !aligned(*t, 16)) return MSS_ERR_LAYOUT;
        for (const mss_tensor_t* t : {x, dt, A, B, C, D, z, dt_bias}) {
            if (overlap(out, t)) return MSS_ERR_ALIAS;
            if (last_state && overlap(last_state, t)) return MSS_ERR_ALIAS;
        }
        if (last_state && overlap(out, last_state)) return MSS_ERR_ALIAS;
        if (x->dtype != MSS_BF16) return MSS_ERR_UNSUPPORTED;        // fp32 inputs: not built
        if (P != 64 || (N != 64 && N != 128)) return MSS_ERR_UNSUPPORTED;
        if (Bt > 65535 || H > 65535) return MSS_ERR_UNSUPPORTED;

        mss::SsdLaunch a;
        a.x = x->data; a.dt = dt->data; a.A = static_cast<const float*>(A->data);
        a.B = B->data; a.C = C->data;
        a.D = D ? static_cast<const float*>(D->data) : nullptr;
        a.z = z ? z->data : nullptr;
        a.bias = dt_bias ? static_cast<const float*>(dt_bias->data) : nullptr;
        a.out = out->data;
        a.last_state = last_state ? static_cast<float*>(last_state->data) : nullptr;
        a.Bt = Bt; a.L = L; a.H = H; a.P = P; a.G = G; a.N = N;
        a.softplus = softplus_flag ? 1 : 0;
        if (Bt * H == 0) return MSS_OK;
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess) return MSS_ERR_HIP;
        if (device_cus(dev, &cus) != hipSuccess) return MSS_ERR_HIP;
        const int segments = mss::plan_ssd_segments(a, cus, g_ssd_segments.load());
        const size_t bytes = mss::ssd_workspace_bytes(a, segments);
        float* ws = nullptr;
        if (bytes > 0) {
            const int wst = workspace(dev, stream, bytes, &ws);
            if (wst != MSS_OK) return wst;
        }
        return mss::launch_ssd_scan(a, segments, ws, static_cast<hipStream_t>(stream)) == hipSuccess ? MSS_OK
                                                                                                    : MSS_ERR_HIP;
    } catch (...) {
        return MSS_ERR_HIP;
    }
}

int mss_release_workspaces(void) {
    try {
        std::lock_guard<std::mutex> lk(g_mu);
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return MSS_ERR_HIP;
        std::vector<std::pair<int, void*>> all(g_retired);
        for (const auto& kv : g_ws)
            if (kv.second.ptr) all.emplace_back(kv.second.dev, kv.second.ptr);
        int st = MSS_OK;
        for (const auto& b : all) {
            if (hipSetDevice(b.first) != hipSuccess || hipDeviceSynchronize() != hipSuccess || hipFree(b.second) != hipSuccess)
                st = MSS_ERR_HIP;
        }
        g_retired.clear();
        g_ws.clear();
        if (hipSetDevice(cur) != hipSuccess) st = MSS_ERR_HIP;
        return st;
    } catch (...) {
        return MSS_ERR_HIP;
    }
}

int mss_set_plan_overrides(int force_generic, int generic_segments, int64_t fast_waves, int bwd_segments,
                           int ssd_segments) {
    if (generic_segments < 0 || fast_waves < 0 || bwd_segments < 0 || ssd_segments < 0) return MSS_ERR_SHAPE;
    g_ssd_segments.store(ssd_segments);
    g_force_generic.store(force_generic != 0 ? 1 : 0);
    g_generic_segments.store(generic_segments);
    g_fast_waves.store(fast_waves);
    g_bwd_segments.store(bwd_segments);
    return MSS_OK;
}

int mss_selective_state_update(const mss_tensor_t* state, const mss_tensor_t* x, const mss_tensor_t* dt,
                               const mss_tensor_t* A, const mss_tensor_t* B, const mss_tensor_t* C,
                               const mss_tensor_t* D, const mss_tensor_t* z, const mss_tensor_t* dt_bias,
                               const mss_tensor_t* out, void* stream) {
    try {
        const int st = validate_decode(state, x, dt, A, B, C, D, z, dt_bias, out);
        if (st != MSS_OK) return st;
        mss::DecodeLaunch a;
        a.state = static_cast<float*>(state->data);
        a.x = x->data; a.dt = dt->data; a.z = z ? z->data : nullptr;
        a.A = static_cast<const float*>(A->data);
        a.B = static_cast<const float*>(B->data);
        a.C = static_cast<const float*>(C->data);
        a.D = D ? static_cast<const float*>(D->data) : nullptr;
        a.bias = dt_bias ? static_cast<const float*>(dt_bias->data) : nullptr;
        a.out = out->data;
        a.Bt = state->shape[0]; a.Dn = state->shape[1]; a.N = static_cast<int>(state->shape[2]);
        a.bf16 = x->dtype == MSS_BF16;
        if (a.Bt * a.Dn == 0) return MSS_OK;
        return mss::launch_state_update(a, static_cast<hipStream_t>(stream)) == hipSuccess ? MSS_OK
                                                                                        : MSS_ERR_HIP;
    } catch (...) {
        return MSS_ERR_HIP;
    }
}

}  // extern "C"
