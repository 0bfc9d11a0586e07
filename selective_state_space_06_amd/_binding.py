"""ctypes binding of libmamba_scan (argument marshalling only; all compute runs in the HIP
kernels behind the C ABI declared in include/mamba_scan.h).

There is no fallback: if the shared library has not been built, loading raises.
"""
from __future__ import annotations

import ctypes
import struct
import os
import threading

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmamba_scan.so")

MSS_F32, MSS_BF16, MSS_I32 = 0, 1, 2
STATUS = {0: "MSS_OK", -1: "MSS_ERR_NULL_ARG", -2: "MSS_ERR_SHAPE", -3: "MSS_ERR_DTYPE",
          -4: "MSS_ERR_LAYOUT", -5: "MSS_ERR_ALIAS", -6: "MSS_ERR_UNSUPPORTED", -7: "MSS_ERR_HIP"}

# every symbol include/mamba_scan.h declares
EXPORTS = ("mss_selective_scan_fwd", "mss_selective_scan_fwd_with_state",
           "mss_selective_scan_fwd_varlen", "mss_selective_scan_bwd", "mss_selective_scan_bwd_varlen",
           "mss_selective_scan_fwd_save", "mss_selective_scan_bwd_saved",
           "mss_selective_state_update", "mss_causal_conv1d_fwd", "mss_causal_conv1d_update", "mss_profile_enable", "mss_profile_fwd",
           "mss_release_workspaces", "mss_set_plan_overrides", "mss_selective_scan_fwd_noalloc",
           "mss_ssd_scan_fwd",
           "mss_status_string", "mss_version")


class Tensor(ctypes.Structure):
    """mss_tensor_t"""
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]

    @classmethod
    def make(cls, data: int, dtype: int, shape, stride=None) -> "Tensor":
        t = cls()
        t.data = data
        t.dtype = dtype
        t.ndim = len(shape)
        if stride is None:
            stride, acc = [], 1
            for s in reversed(shape):
                stride.insert(0, acc)
                acc *= s
        for i, (s, st) in enumerate(zip(shape[:4], stride[:4])):  # ndim > 4: rejected by the ABI
            t.shape[i] = s
            t.stride[i] = st
        return t


_TP = ctypes.POINTER(Tensor)
_lib = None
_lock = threading.Lock()


class MssError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed: {STATUS.get(status, status)}")


def load_library(path: str = LIB_PATH):
    """Load libmamba_scan.so; raises if it is missing (build it first)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError(
                    f"{path} is missing: build it with `python -m selective_state_space_06_amd.build` "
                    "or __graft_entry__.build(); there is no fallback implementation")
            # torch's ROCm wheel carries its own libamdhip64.so: load it first, so that this
            # library binds to the HIP runtime torch's streams and allocations belong to (loaded
            # first itself, it would pull in /opt/rocm's copy, and a second runtime in the process
            # rejects torch's stream handles at launch)
            try:
                import torch  # noqa: F401
            except ImportError:
                pass
            lib = ctypes.CDLL(path)
            lib.mss_selective_scan_fwd.restype = ctypes.c_int
            lib.mss_selective_scan_fwd.argtypes = [_TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP,
                                                   ctypes.c_int, _TP, _TP, ctypes.c_void_p]
            lib.mss_selective_scan_fwd_with_state.restype = ctypes.c_int
            lib.mss_selective_scan_fwd_with_state.argtypes = [
                _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, ctypes.c_int, _TP, _TP, ctypes.c_void_p]
            lib.mss_selective_scan_fwd_varlen.restype = ctypes.c_int
            lib.mss_selective_scan_fwd_varlen.argtypes = [
                _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, ctypes.c_int, _TP, _TP, ctypes.c_void_p]
            lib.mss_selective_scan_bwd.restype = ctypes.c_int
            lib.mss_selective_scan_bwd.argtypes = [
                _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, ctypes.c_int, _TP,
                _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, ctypes.c_void_p]
            lib.mss_causal_conv1d_fwd.restype = ctypes.c_int
            lib.mss_causal_conv1d_fwd.argtypes = [_TP, _TP, _TP, _TP, ctypes.c_int, _TP, _TP,
                                                  ctypes.c_void_p]
            lib.mss_causal_conv1d_update.restype = ctypes.c_int
            lib.mss_causal_conv1d_update.argtypes = [_TP, _TP, _TP, _TP, ctypes.c_int, _TP,
                                                     ctypes.c_void_p]
            lib.mss_selective_scan_bwd_varlen.restype = ctypes.c_int
            lib.mss_selective_scan_bwd_varlen.argtypes = [
                _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, ctypes.c_int, _TP, _TP,
                _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, ctypes.c_void_p]
            lib.mss_selective_scan_fwd_save.restype = ctypes.c_int
            lib.mss_selective_scan_fwd_save.argtypes = [
                _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, ctypes.c_int, _TP, _TP, _TP,
                ctypes.c_void_p]
            lib.mss_selective_scan_bwd_saved.restype = ctypes.c_int
            lib.mss_selective_scan_bwd_saved.argtypes = [
                _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, ctypes.c_int, _TP, _TP, _TP,
                _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, ctypes.c_void_p]
            lib.mss_selective_state_update.restype = ctypes.c_int
            lib.mss_selective_state_update.argtypes = [_TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP,
                                                       _TP, _TP, ctypes.c_void_p]
            lib.mss_status_string.restype = ctypes.c_char_p
            lib.mss_status_string.argtypes = [ctypes.c_int]
            lib.mss_version.restype = ctypes.c_int
            lib.mss_version.argtypes = []
            lib.mss_selective_scan_fwd_noalloc.restype = ctypes.c_int
            lib.mss_selective_scan_fwd_noalloc.argtypes = [_TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP,
                                                           ctypes.c_int, _TP, _TP, ctypes.c_void_p]
            lib.mss_ssd_scan_fwd.restype = ctypes.c_int
            lib.mss_ssd_scan_fwd.argtypes = [_TP, _TP, _TP, _TP, _TP, _TP, _TP, _TP, ctypes.c_int, _TP, _TP,
                                             ctypes.c_void_p]
            lib.mss_release_workspaces.restype = ctypes.c_int
            lib.mss_release_workspaces.argtypes = []
            lib.mss_set_plan_overrides.restype = ctypes.c_int
            lib.mss_set_plan_overrides.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                                   ctypes.c_int]
            lib.mss_profile_enable.restype = ctypes.c_int
            lib.mss_profile_enable.argtypes = [ctypes.c_int]
            lib.mss_profile_fwd.restype = ctypes.c_int
            lib.mss_profile_fwd.argtypes = [ctypes.POINTER(ctypes.c_int),
                                            ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(ctypes.c_double)]
            _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load_library().mss_status_string(int(status)).decode()


def version() -> int:
    return int(load_library().mss_version())


def release_workspaces() -> None:
    """mss_release_workspaces: free the library's workspace buffers (after the device is idle)."""
    st = load_library().mss_release_workspaces()
    if st != 0:
        raise MssError(st, "mss_release_workspaces")


def set_plan_overrides(force_generic: bool = False, generic_segments: int = 0, fast_waves: int = 0,
                       bwd_segments: int = 0, ssd_segments: int = 0) -> None:
    """mss_set_plan_overrides (tests and tuning only): fix the forward's path and split, the
    backward's and the SSD scan's segment counts for later calls; all defaults restore the
    automatic plans."""
    st = load_library().mss_set_plan_overrides(1 if force_generic else 0, int(generic_segments),
                                                int(fast_waves), int(bwd_segments), int(ssd_segments))
    if st != 0:
        raise MssError(st, "mss_set_plan_overrides")


def profile_enable(on: bool = True) -> None:
    """mss_profile_enable: record launch-timing events around each forward scan's kernels."""
    st = load_library().mss_profile_enable(1 if on else 0)
    if st != 0:
        raise MssError(st, "mss_profile_enable")


def profile_fwd():
    """mss_profile_fwd: (calls, carry_ms_total, main_ms_total) of the recorded forward scans."""
    n, c, m = ctypes.c_int(), ctypes.c_double(), ctypes.c_double()
    st = load_library().mss_profile_fwd(ctypes.byref(n), ctypes.byref(c), ctypes.byref(m))
    if st != 0:
        raise MssError(st, "mss_profile_fwd")
    return int(n.value), float(c.value), float(m.value)


def _ref(t):
    return None if t is None else ctypes.byref(t)


def scan_fwd_raw(u, delta, A, B, C, D, z, delta_bias, softplus_flag, out, last_state, stream) -> int:
    """Direct call of mss_selective_scan_fwd with Tensor descriptors (or None)."""
    return load_library().mss_selective_scan_fwd(
        _ref(u), _ref(delta), _ref(A), _ref(B), _ref(C), _ref(D), _ref(z), _ref(delta_bias),
        int(softplus_flag), _ref(out), _ref(last_state), stream)


def scan_fwd_noalloc_raw(u, delta, A, B, C, D, z, delta_bias, softplus_flag, out, last_state, stream) -> int:
    return load_library().mss_selective_scan_fwd_noalloc(_ref(u), _ref(delta), _ref(A), _ref(B), _ref(C), _ref(D),
                                                         _ref(z), _ref(delta_bias), int(softplus_flag), _ref(out),
                                                         _ref(last_state), stream)


def ssd_scan_fwd_raw(x, dt, A, B, C, D, z, dt_bias, softplus_flag, out, last_state, stream) -> int:
    return load_library().mss_ssd_scan_fwd(_ref(x), _ref(dt), _ref(A), _ref(B), _ref(C), _ref(D), _ref(z),
                                           _ref(dt_bias), int(softplus_flag), _ref(out), _ref(last_state), stream)


def scan_fwd_with_state_raw(u, delta, A, B, C, D, z, delta_bias, initial_state, softplus_flag,
                            out, last_state, stream) -> int:
    """Direct call of mss_selective_scan_fwd_with_state with Tensor descriptors (or None)."""
    return load_library().mss_selective_scan_fwd_with_state(
        _ref(u), _ref(delta), _ref(A), _ref(B), _ref(C), _ref(D), _ref(z), _ref(delta_bias),
        _ref(initial_state), int(softplus_flag), _ref(out), _ref(last_state), stream)


def scan_fwd_varlen_raw(u, delta, A, B, C, D, z, delta_bias, initial_state, seq_lens, softplus_flag,
                        out, last_state, stream) -> int:
    """Direct call of mss_selective_scan_fwd_varlen with Tensor descriptors (or None)."""
    return load_library().mss_selective_scan_fwd_varlen(
        _ref(u), _ref(delta), _ref(A), _ref(B), _ref(C), _ref(D), _ref(z), _ref(delta_bias),
        _ref(initial_state), _ref(seq_lens), int(softplus_flag), _ref(out), _ref(last_state), stream)


def scan_bwd_raw(u, delta, A, B, C, D, z, delta_bias, softplus_flag, dout, du, ddelta, dA, dB, dC,
                 dD, dz, ddelta_bias, stream) -> int:
    """Direct call of mss_selective_scan_bwd with Tensor descriptors (or None)."""
    return load_library().mss_selective_scan_bwd(
        _ref(u), _ref(delta), _ref(A), _ref(B), _ref(C), _ref(D), _ref(z), _ref(delta_bias),
        int(softplus_flag), _ref(dout), _ref(du), _ref(ddelta), _ref(dA), _ref(dB), _ref(dC),
        _ref(dD), _ref(dz), _ref(ddelta_bias), stream)


def scan_bwd_varlen_raw(u, delta, A, B, C, D, z, delta_bias, initial_state, seq_lens, softplus_flag,
                        dout, dlast_state, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias,
                        dinitial_state, stream) -> int:
    """Direct call of mss_selective_scan_bwd_varlen with Tensor descriptors (or None)."""
    return load_library().mss_selective_scan_bwd_varlen(
        _ref(u), _ref(delta), _ref(A), _ref(B), _ref(C), _ref(D), _ref(z), _ref(delta_bias),
        _ref(initial_state), _ref(seq_lens), int(softplus_flag), _ref(dout), _ref(dlast_state),
        _ref(du), _ref(ddelta), _ref(dA), _ref(dB), _ref(dC), _ref(dD), _ref(dz),
        _ref(ddelta_bias), _ref(dinitial_state), stream)


def scan_fwd_save_raw(u, delta, A, B, C, D, z, delta_bias, initial_state, seq_lens, softplus_flag,
                      out, last_state, saved_states, stream) -> int:
    """Direct call of mss_selective_scan_fwd_save with Tensor descriptors (or None)."""
    return load_library().mss_selective_scan_fwd_save(
        _ref(u), _ref(delta), _ref(A), _ref(B), _ref(C), _ref(D), _ref(z), _ref(delta_bias),
        _ref(initial_state), _ref(seq_lens), int(softplus_flag), _ref(out), _ref(last_state),
        _ref(saved_states), stream)


def scan_bwd_saved_raw(u, delta, A, B, C, D, z, delta_bias, seq_lens, softplus_flag, saved_states,
                       dout, dlast_state, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias,
                       dinitial_state, stream) -> int:
    """Direct call of mss_selective_scan_bwd_saved with Tensor descriptors (or None)."""
    return load_library().mss_selective_scan_bwd_saved(
        _ref(u), _ref(delta), _ref(A), _ref(B), _ref(C), _ref(D), _ref(z), _ref(delta_bias),
        _ref(seq_lens), int(softplus_flag), _ref(saved_states), _ref(dout), _ref(dlast_state),
        _ref(du), _ref(ddelta), _ref(dA), _ref(dB), _ref(dC), _ref(dD), _ref(dz),
        _ref(ddelta_bias), _ref(dinitial_state), stream)


def conv1d_fwd_raw(x, weight, bias, initial_state, silu_flag, out, final_state, stream) -> int:
    """Direct call of mss_causal_conv1d_fwd with Tensor descriptors (or None)."""
    return load_library().mss_causal_conv1d_fwd(
        _ref(x), _ref(weight), _ref(bias), _ref(initial_state), int(silu_flag), _ref(out),
        _ref(final_state), stream)


def conv1d_update_raw(state, x, weight, bias, silu_flag, out, stream) -> int:
    """Direct call of mss_causal_conv1d_update with Tensor descriptors (or None)."""
    return load_library().mss_causal_conv1d_update(
        _ref(state), _ref(x), _ref(weight), _ref(bias), int(silu_flag), _ref(out), stream)


def state_update_raw(state, x, dt, A, B, C, D, z, dt_bias, out, stream) -> int:
    """Direct call of mss_selective_state_update with Tensor descriptors (or None)."""
    return load_library().mss_selective_state_update(
        _ref(state), _ref(x), _ref(dt), _ref(A), _ref(B), _ref(C), _ref(D), _ref(z),
        _ref(dt_bias), _ref(out), stream)


# ----------------------------------------------------------------------- torch front end

_DESC = struct.Struct("<Qii4q4q")   # the bytes of one Tensor (mss_tensor_t)
_DTYPES = None


def _desc(t):
    """torch tensor (or None) -> Tensor descriptor, packed in one step (this runs for every
    argument of every call, so it is kept to a few attribute reads)."""
    global _DTYPES
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmamba_scan takes device tensors")
    if _DTYPES is None:
        import torch
        _DTYPES = {torch.float32: MSS_F32, torch.bfloat16: MSS_BF16, torch.int32: MSS_I32}
    shape, stride = tuple(t.shape), t.stride()
    n = len(shape)
    if n > 4:
        return Tensor.make(t.data_ptr(), _DTYPES.get(t.dtype, -1), list(shape), list(stride))  # rejected by the ABI
    pad = (0,) * (4 - n)
    return Tensor.from_buffer_copy(_DESC.pack(t.data_ptr(), _DTYPES.get(t.dtype, -1), n, *shape, *pad,
                                              *stride, *pad))


def _stream_of(dev_):
    """The current HIP stream of dev_ (an int) when dev_ is the current device, else None (the
    caller then switches devices for the call)."""
    import torch
    if dev_.index is None or dev_.index == torch.cuda.current_device():
        return torch.cuda.current_stream().cuda_stream
    return None


def selective_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                       return_last_state=True, out=None, last_state=None):
    """Forward selective scan on the current stream of u's device.

    u, delta, z: (batch, d_inner, L) float32 or bfloat16; A: (d_inner, d_state) float32;
    B, C: (batch, d_state, L) float32; D, delta_bias: (d_inner,) float32; d_state 16, 32, 64 or
    128.  Returns out (dtype of u), or (out, last_state) with last_state (batch, d_inner, d_state)
    float32.
    """
    import torch
    if out is None:
        out = torch.empty_like(u, memory_format=torch.contiguous_format)
    if return_last_state and last_state is None:
        last_state = torch.empty((u.shape[0], u.shape[1], A.shape[1]), dtype=torch.float32,
                                 device=u.device)
    with torch.cuda.device(u.device):
        stream = torch.cuda.current_stream(u.device).cuda_stream
        st = scan_fwd_raw(_desc(u), _desc(delta), _desc(A), _desc(B), _desc(C), _desc(D), _desc(z),
                          _desc(delta_bias), 1 if delta_softplus else 0, _desc(out),
                          _desc(last_state) if return_last_state else None, stream)
    if st != 0:
        raise MssError(st, "mss_selective_scan_fwd")
    return (out, last_state) if return_last_state else out



def selective_scan_fwd_noalloc(u, delta, A, B, C, out, D=None, z=None, delta_bias=None,
                               delta_softplus=True, last_state=None):
    """mss_selective_scan_fwd_noalloc on the current stream of u's device: the forward scan with
    the library's fixed per-GPU scratch (no device allocation by the library).  The caller passes
    `out` (and `last_state`, or None): this wrapper allocates nothing either."""
    import torch
    with torch.cuda.device(u.device):
        stream = torch.cuda.current_stream(u.device).cuda_stream
        st = scan_fwd_noalloc_raw(_desc(u), _desc(delta), _desc(A), _desc(B), _desc(C), _desc(D), _desc(z),
                                  _desc(delta_bias), 1 if delta_softplus else 0, _desc(out), _desc(last_state),
                                  stream)
    if st != 0:
        raise MssError(st, "mss_selective_scan_fwd_noalloc")
    return out

def causal_conv1d_fwd(x, weight, bias=None, initial_state=None, silu=True, out=None,
                      return_final_state=False, final_state=None):
    """Causal depthwise conv1d (+ silu) on the current stream.  x: (batch, d_inner, L) float32
    or bfloat16; weight: (d_inner, K) float32, K <= 4; bias: (d_inner,) float32; initial_state:
    (batch, d_inner, K - 1) in x's dtype.  Returns out, or (out, final_state)."""
    import torch
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    if return_final_state and final_state is None:
        final_state = torch.empty((x.shape[0], x.shape[1], weight.shape[1] - 1), dtype=x.dtype,
                                  device=x.device)
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        st = conv1d_fwd_raw(_desc(x), _desc(weight), _desc(bias), _desc(initial_state),
                            1 if silu else 0, _desc(out),
                            _desc(final_state) if return_final_state else None, stream)
    if st != 0:
        raise MssError(st, "mss_causal_conv1d_fwd")
    return (out, final_state) if return_final_state else out


def causal_conv1d_update(state, x, weight, bias=None, silu=True, out=None):
    """One token of the conv per row; `state` (batch, d_inner, K - 1) in x's dtype is updated in
    place.  x: (batch, d_inner).  Returns out (batch, d_inner)."""
    import torch
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    stream = _stream_of(x.device)
    if stream is not None:
        st = conv1d_update_raw(_desc(state), _desc(x), _desc(weight), _desc(bias), 1 if silu else 0,
                               _desc(out), stream)
    else:
        with torch.cuda.device(x.device):
            stream = torch.cuda.current_stream(x.device).cuda_stream
            st = conv1d_update_raw(_desc(state), _desc(x), _desc(weight), _desc(bias),
                                   1 if silu else 0, _desc(out), stream)
    if st != 0:
        raise MssError(st, "mss_causal_conv1d_update")
    return out


def selective_scan_bwd(u, delta, A, B, C, dout, D=None, z=None, delta_bias=None,
                       delta_softplus=True, initial_state=None, seq_lens=None, dlast_state=None,
                       return_dinitial_state=False, saved_states=None):
    """Gradients of selective_scan_fwd (from h = 0) for L = sum(dout * out), on the current
    stream.  Returns a dict: du, ddelta, dz (None without z) in u's dtype; dA, dB, dC, dD,
    ddelta_bias in float32 (dD / ddelta_bias also when D / delta_bias is None).
    initial_state / seq_lens describe the forward (as selective_scan_fwd_varlen); dlast_state is
    dL/d last_state; with return_dinitial_state the dict also holds dinitial_state = dL/dh0.
    saved_states: the states selective_scan_fwd_save wrote for this forward (it carries the
    forward's initial_state); the backward then reads them instead of recomputing them."""
    import torch
    dev_ = u.device
    Bt, Dn, L = u.shape
    N = A.shape[1]
    f32 = dict(dtype=torch.float32, device=dev_)
    g = dict(du=torch.empty((Bt, Dn, L), dtype=u.dtype, device=dev_),
             ddelta=torch.empty((Bt, Dn, L), dtype=u.dtype, device=dev_),
             dz=None if z is None else torch.empty((Bt, Dn, L), dtype=u.dtype, device=dev_),
             dA=torch.empty((Dn, N), **f32), dB=torch.empty((Bt, N, L), **f32),
             dC=torch.empty((Bt, N, L), **f32), dD=torch.empty((Dn,), **f32),
             ddelta_bias=torch.empty((Dn,), **f32))
    if return_dinitial_state:
        g["dinitial_state"] = torch.empty((Bt, Dn, N), **f32)
    with torch.cuda.device(dev_):
        stream = torch.cuda.current_stream(dev_).cuda_stream
        if saved_states is not None:
            st = scan_bwd_saved_raw(_desc(u), _desc(delta), _desc(A), _desc(B), _desc(C), _desc(D),
                                    _desc(z), _desc(delta_bias), _desc(seq_lens),
                                    1 if delta_softplus else 0, _desc(saved_states), _desc(dout),
                                    _desc(dlast_state), _desc(g["du"]), _desc(g["ddelta"]),
                                    _desc(g["dA"]), _desc(g["dB"]), _desc(g["dC"]), _desc(g["dD"]),
                                    _desc(g["dz"]), _desc(g["ddelta_bias"]),
                                    _desc(g.get("dinitial_state")), stream)
            if st != 0:
                raise MssError(st, "mss_selective_scan_bwd_saved")
            return g
        st = scan_bwd_varlen_raw(_desc(u), _desc(delta), _desc(A), _desc(B), _desc(C), _desc(D),
                                 _desc(z), _desc(delta_bias), _desc(initial_state),
                                 _desc(seq_lens), 1 if delta_softplus else 0, _desc(dout),
                                 _desc(dlast_state), _desc(g["du"]), _desc(g["ddelta"]),
                                 _desc(g["dA"]), _desc(g["dB"]), _desc(g["dC"]), _desc(g["dD"]),
                                 _desc(g["dz"]), _desc(g["ddelta_bias"]),
                                 _desc(g.get("dinitial_state")), stream)
    if st != 0:
        raise MssError(st, "mss_selective_scan_bwd_varlen")
    return g


class SelectiveScanFunction:
    """torch.autograd wrapper: out = selective_scan_fwd(...) with gradients from the library's
    backward.  save_states=True keeps the forward's states at every eighth step (8 bytes per
    (batch, d_inner, step)) for the backward; False recomputes them there.  Marshalling only:
    both passes run in the library's kernels.  Usage: SelectiveScanFunction.apply(u, delta, A, B,
    C, D, z, delta_bias, delta_softplus, save_states); D, z, delta_bias may be None."""

    _fn = None

    @classmethod
    def apply(cls, u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
              save_states=False):
        if cls._fn is None:
            cls._fn = _make_autograd_fn()
        return cls._fn.apply(u, delta, A, B, C, D, z, delta_bias, delta_softplus, save_states)


def _make_autograd_fn():
    import torch

    class _Fn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, u, delta, A, B, C, D, z, delta_bias, delta_softplus, save_states):
            saved = None
            if save_states:
                out, _, saved = selective_scan_fwd_save(u, delta, A, B, C, D=D, z=z,
                                                        delta_bias=delta_bias,
                                                        delta_softplus=delta_softplus)
            else:
                out = selective_scan_fwd(u, delta, A, B, C, D=D, z=z, delta_bias=delta_bias,
                                         delta_softplus=delta_softplus, return_last_state=False)
            ctx.save_for_backward(u, delta, A, B, C, D, z, delta_bias, saved)
            ctx.delta_softplus = delta_softplus
            return out

        @staticmethod
        def backward(ctx, dout):
            u, delta, A, B, C, D, z, delta_bias, saved = ctx.saved_tensors
            g = selective_scan_bwd(u, delta, A, B, C, dout.contiguous(), D=D, z=z,
                                   delta_bias=delta_bias, delta_softplus=ctx.delta_softplus,
                                   saved_states=saved)
            return (g["du"], g["ddelta"], g["dA"], g["dB"], g["dC"],
                    g["dD"] if D is not None else None, g["dz"],
                    g["ddelta_bias"] if delta_bias is not None else None, None, None)

    return _Fn


def selective_scan_fwd_varlen(u, delta, A, B, C, seq_lens, initial_state=None, D=None, z=None,
                              delta_bias=None, delta_softplus=True, out=None, last_state=None):
    """Forward scan of sequences of different lengths: seq_lens (batch,) int32 on the device.
    Outputs past a sequence's end are 0; last_state[b] is the state after step seq_lens[b] - 1.
    Returns (out, last_state)."""
    import torch
    if out is None:
        out = torch.empty_like(u, memory_format=torch.contiguous_format)
    if last_state is None:
        last_state = torch.empty((u.shape[0], u.shape[1], A.shape[1]), dtype=torch.float32,
                                 device=u.device)
    with torch.cuda.device(u.device):
        stream = torch.cuda.current_stream(u.device).cuda_stream
        st = scan_fwd_varlen_raw(_desc(u), _desc(delta), _desc(A), _desc(B), _desc(C), _desc(D),
                                 _desc(z), _desc(delta_bias), _desc(initial_state), _desc(seq_lens),
                                 1 if delta_softplus else 0, _desc(out), _desc(last_state), stream)
    if st != 0:
        raise MssError(st, "mss_selective_scan_fwd_varlen")
    return out, last_state


def selective_scan_fwd_save(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                            initial_state=None, seq_lens=None, out=None, last_state=None,
                            saved_states=None):
    """Forward scan (as selective_scan_fwd_varlen; seq_lens and initial_state may be None) that
    also writes the states its backward reads: saved_states (ceil(L / 8), 4, batch * d_inner * 4)
    float32, the state entering every eighth step (state n of row r entering step 8k at
    [k, n // 4, 4 r + n % 4]; saved_state_blocks() gives (ceil(L / 8), batch * d_inner, 16)).
    Returns (out, last_state, saved_states)."""
    import torch
    Bt, Dn, L = u.shape
    if out is None:
        out = torch.empty_like(u, memory_format=torch.contiguous_format)
    if last_state is None:
        last_state = torch.empty((Bt, Dn, A.shape[1]), dtype=torch.float32, device=u.device)
    if saved_states is None:
        saved_states = torch.empty(((L + 7) // 8, A.shape[1] // 4, Bt * Dn * 4),
                                   dtype=torch.float32, device=u.device)
    with torch.cuda.device(u.device):
        stream = torch.cuda.current_stream(u.device).cuda_stream
        st = scan_fwd_save_raw(_desc(u), _desc(delta), _desc(A), _desc(B), _desc(C), _desc(D),
                               _desc(z), _desc(delta_bias), _desc(initial_state), _desc(seq_lens),
                               1 if delta_softplus else 0, _desc(out), _desc(last_state),
                               _desc(saved_states), stream)
    if st != 0:
        raise MssError(st, "mss_selective_scan_fwd_save")
    return out, last_state, saved_states


def saved_state_blocks(saved_states):
    """View of selective_scan_fwd_save's saved_states as (ceil(L / 8), batch * d_inner, 16): block
    k is the state entering step 8k, laid out like last_state (a copy; for inspection)."""
    K, Q, R4 = saved_states.shape
    return saved_states.reshape(K, Q, R4 // 4, 4).permute(0, 2, 1, 3).reshape(K, R4 // 4, 4 * Q)


def selective_scan_fwd_with_state(u, delta, A, B, C, initial_state, D=None, z=None,
                                  delta_bias=None, delta_softplus=True, out=None, last_state=None):
    """Forward selective scan continued from `initial_state` (batch, d_inner, d_state) float32
    (None: from zeros).  Other arguments as selective_scan_fwd; returns (out, last_state).
    last_state must be a different buffer from initial_state."""
    import torch
    if out is None:
        out = torch.empty_like(u, memory_format=torch.contiguous_format)
    if last_state is None:
        last_state = torch.empty((u.shape[0], u.shape[1], A.shape[1]), dtype=torch.float32,
                                 device=u.device)
    with torch.cuda.device(u.device):
        stream = torch.cuda.current_stream(u.device).cuda_stream
        st = scan_fwd_with_state_raw(_desc(u), _desc(delta), _desc(A), _desc(B), _desc(C),
                                     _desc(D), _desc(z), _desc(delta_bias), _desc(initial_state),
                                     1 if delta_softplus else 0, _desc(out), _desc(last_state),
                                     stream)
    if st != 0:
        raise MssError(st, "mss_selective_scan_fwd_with_state")
    return out, last_state


def selective_state_update(state, x, dt, A, B, C, D=None, z=None, dt_bias=None, out=None):
    """One decode step on the current stream; `state` (batch, d_inner, d_state) float32 is updated
    in place, d_state 16, 32, 64 or 128.  x, dt, z: (batch, d_inner) float32 or bfloat16; B, C:
    (batch, d_state) float32.
    Returns out (batch, d_inner) in x's dtype."""
    import torch
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    stream = _stream_of(x.device)
    if stream is not None:
        st = state_update_raw(_desc(state), _desc(x), _desc(dt), _desc(A), _desc(B), _desc(C),
                              _desc(D), _desc(z), _desc(dt_bias), _desc(out), stream)
    else:
        with torch.cuda.device(x.device):
            stream = torch.cuda.current_stream(x.device).cuda_stream
            st = state_update_raw(_desc(state), _desc(x), _desc(dt), _desc(A), _desc(B), _desc(C),
                                  _desc(D), _desc(z), _desc(dt_bias), _desc(out), stream)
    if st != 0:
        raise MssError(st, "mss_selective_state_update")
    return out


def _bound_stream(x, stream):
    import torch
    if not x.is_cuda:
        raise ValueError("libmamba_scan takes device tensors")
    if stream is None:
        with torch.cuda.device(x.device):
            return torch.cuda.current_stream(x.device).cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


class StateUpdateStep:
    """mss_selective_state_update bound to fixed device buffers, for decode loops that refill the
    same input buffers every token: the argument descriptors and the stream are taken once, here,
    so each call costs one foreign-function call (the library still validates every call).
    Arguments as for selective_state_update; `stream` defaults to the current stream of x's
    device at construction.  The object keeps its tensors alive; calling it updates `state` in
    place and writes `out` (returned)."""

    def __init__(self, state, x, dt, A, B, C, D=None, z=None, dt_bias=None, out=None, stream=None):
        import torch
        stream = _bound_stream(x, stream)
        if out is None:
            out = torch.empty_like(x, memory_format=torch.contiguous_format)
        self.out = out
        self._keep = (state, x, dt, A, B, C, D, z, dt_bias, out)
        self._descs = [_desc(t) for t in self._keep]
        self._args = tuple(_ref(d) for d in self._descs) + (stream,)
        self._fn = load_library().mss_selective_state_update

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            raise MssError(st, "mss_selective_state_update")
        return self.out


class Conv1dUpdateStep:
    """mss_causal_conv1d_update bound to fixed device buffers (the one-token conv of a decode loop,
    in front of StateUpdateStep): descriptors and stream taken once, here.  Arguments as for
    causal_conv1d_update; calling it shifts `state` in place and writes `out` (returned)."""

    def __init__(self, state, x, weight, bias=None, silu=True, out=None, stream=None):
        import torch
        stream = _bound_stream(x, stream)
        if out is None:
            out = torch.empty_like(x, memory_format=torch.contiguous_format)
        self.out = out
        self._keep = (state, x, weight, bias, out)
        d = [_desc(t) for t in self._keep]
        self._descs = d
        self._args = (_ref(d[0]), _ref(d[1]), _ref(d[2]), _ref(d[3]), 1 if silu else 0, _ref(d[4]), stream)
        self._fn = load_library().mss_causal_conv1d_update

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            raise MssError(st, "mss_causal_conv1d_update")
        return self.out


def ssd_scan_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=True, return_last_state=True,
                 out=None, last_state=None):
    """Mamba-2 SSD layer (mss_ssd_scan_fwd) on the current stream of x's device.

    x, z: (batch, L, heads, 64) bfloat16; dt: (batch, L, heads) bfloat16; A, D, dt_bias: (heads,)
    float32; B, C: (batch, L, groups, d_state) bfloat16 with d_state 64 or 128.
    Returns out, or (out, last_state) with last_state (batch, heads, 64, d_state) float32.
    """
    import torch
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    if return_last_state and last_state is None:
        last_state = torch.empty((x.shape[0], x.shape[2], x.shape[3], B.shape[3]), dtype=torch.float32,
                                 device=x.device)
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        st = ssd_scan_fwd_raw(_desc(x), _desc(dt), _desc(A), _desc(B), _desc(C), _desc(D), _desc(z),
                              _desc(dt_bias), 1 if dt_softplus else 0, _desc(out),
                              _desc(last_state) if return_last_state else None, stream)
    if st != 0:
        raise MssError(st, "mss_ssd_scan_fwd")
    return (out, last_state) if return_last_state else out
