"""Python binding of liblinattn: normalized kernelized linear attention on AMD MI355X.

A thin ctypes layer over the C ABI in ``include/la.h``: it only reads tensor shapes, data
pointers and the current HIP stream and passes them on. Every step of the computation runs in
the library's HIP kernels. PyTorch supplies device memory and streams; nothing else.

The entry points keep the C names:
    la_causal_fwd(q, k, v, out, S=None, z=None, chunk=0, seg_len=0)
    la_causal_fwd_ex(q, k, v, out, S0=None, z0=None, S=None, z=None, chunk=0, seg_len=0, flags=0)
    la_global_fwd(q, k, v, out, S, z, chunk=0)         # q, out may be None: state only
    la_global_fwd_ex(q, k, v, out, S, z, chunk=0, flags=0)
    la_decode_step(q, k, v, out, S, z)
    la_decode_step_ex(q, k, v, out, S, z, flags=0)
    la_causal_fwd_decay(q, k, v, out, gamma, S0=None, z0=None, S=None, z=None, chunk=0,
                        seg_len=0, flags=0)            # per-head decay gamma [H] (retention)
    la_decode_step_decay(q, k, v, out, S, z, gamma, flags=0)
    la_rf_features(x, W, f)                            # positive random features
    la_causal_fwd_rf(q, k, v, out, W, S0=None, z0=None, S=None, z=None, chunk=0, seg_len=0,
                     flags=0)                          # causal over random features of q, k
    la_causal_fwd_ws(q, k, v, out, ws, S0=None, z0=None, S=None, z=None, gamma=None, chunk=0,
                     seg_len=0, flags=0)               # caller-supplied workspace ws
    la_global_fwd_ws(q, k, v, out, S, z, ws, chunk=0, flags=0)
    la_causal_fwd_noalloc(q, k, v, out, S0=None, z0=None, S=None, z=None, chunk=0, seg_len=0,
                          flags=0)                     # static scratch: allocates nothing
    la_release_cache()                                 # frees the library's cached scratch
with q, k [B,H,N,d], v, out [B,H,N,d_v] (bf16 or float32, contiguous, on the GPU),
S [B,H,d,d_v] and z [B,H,d] float32; flags is a bitwise or of LA_PHI_IDENTITY and
LA_UNNORMALIZED. A non-zero status raises ``LAError``.

If the shared library is missing or fails to load, importing this package raises: there is
no fallback implementation.

PyTorch ships its own copy of the HIP runtime. The library links the system one by soname, so
PyTorch is imported first: the loader then binds the library to the runtime already in the
process and one runtime serves both (two copies in one process do not share devices, memory
or streams). ``hip_runtimes()`` lists the HIP runtime copies mapped into the process.
"""
from __future__ import annotations

import ctypes
import functools
import os
from pathlib import Path

import torch  # noqa: F401  (must precede loading liblinattn; see above)

_PKG = Path(__file__).resolve().parent
LIB_PATH = Path(os.environ.get("LINATTN_LIB", _PKG / "liblinattn.so"))

LA_F32, LA_BF16 = 0, 1
LA_OK, LA_EINVAL, LA_ENOTSUP, LA_EHIP, LA_ENOSPACE = 0, 1, 2, 3, 4
LA_PHI_IDENTITY, LA_UNNORMALIZED = 1, 2

# Every symbol include/la.h declares.
EXPORTS = ("la_causal_fwd", "la_causal_fwd_seg", "la_causal_fwd_state", "la_causal_fwd_ex",
           "la_causal_fwd_profiled", "la_global_fwd", "la_global_fwd_ex", "la_decode_step",
           "la_decode_step_ex", "la_causal_fwd_decay", "la_decode_step_decay", "la_rf_features",
           "la_causal_fwd_rf", "la_causal_fwd_ws", "la_global_fwd_ws", "la_causal_fwd_noalloc",
           "la_release_cache",
           "la_workspace_bytes", "la_segments", "la_strerror", "la_version")


class LAError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: status {status}: {strerror(status)}")


def _load(path: Path):
    if not path.exists():
        raise ImportError(f"liblinattn not built: {path} is missing "
                          "(run python causal_linear_attention_la_amd/build.py)")
    lib = ctypes.CDLL(str(path))
    vp, fp, i = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
    core = [vp, vp, vp, vp, fp, fp, i, i, i, i, i, i]
    lib.la_causal_fwd.argtypes = core + [i, vp]
    lib.la_causal_fwd_seg.argtypes = core + [i, i, vp]
    state = [vp, vp, vp, vp, fp, fp, fp, fp, i, i, i, i, i, i, i]
    lib.la_causal_fwd_state.argtypes = state + [i, vp]
    lib.la_causal_fwd_ex.argtypes = state + [i, i, vp]
    lib.la_causal_fwd_profiled.argtypes = state + [i, i, vp, i, ctypes.POINTER(ctypes.c_float)]
    lib.la_global_fwd.argtypes = core + [i, vp]
    lib.la_global_fwd_ex.argtypes = core + [i, i, vp]
    lib.la_decode_step.argtypes = core + [i, vp]
    lib.la_decode_step_ex.argtypes = core + [i, vp]
    lib.la_rf_features.argtypes = [vp, vp, vp, ctypes.c_long, i, i, i, vp]
    lib.la_causal_fwd_decay.argtypes = [vp, vp, vp, vp, fp, fp, fp, fp, fp] + [i] * 9 + [vp]
    lib.la_decode_step_decay.argtypes = [vp, vp, vp, vp, fp, fp, fp] + [i] * 7 + [vp]
    lib.la_causal_fwd_rf.argtypes = [vp, vp, vp, vp, vp, fp, fp, fp, fp] + [i] * 10 + [vp]
    sz = ctypes.c_size_t
    lib.la_causal_fwd_ws.argtypes = [vp, vp, vp, vp, fp, fp, fp, fp, fp] + [i] * 9 + [vp, sz, vp]
    lib.la_global_fwd_ws.argtypes = core + [i, i, vp, sz, vp]
    lib.la_causal_fwd_noalloc.argtypes = state + [i, i, vp]
    lib.la_release_cache.argtypes = []
    for f in ("la_causal_fwd", "la_causal_fwd_seg", "la_causal_fwd_state", "la_causal_fwd_ex",
              "la_causal_fwd_profiled", "la_global_fwd", "la_global_fwd_ex", "la_decode_step",
              "la_decode_step_ex", "la_rf_features", "la_causal_fwd_decay", "la_decode_step_decay",
              "la_causal_fwd_rf", "la_causal_fwd_ws", "la_global_fwd_ws", "la_causal_fwd_noalloc",
              "la_release_cache"):
        getattr(lib, f).restype = ctypes.c_int
    lib.la_workspace_bytes.argtypes = [i] * 8 + [i]
    lib.la_workspace_bytes.restype = ctypes.c_size_t
    lib.la_segments.argtypes = [i] * 9
    lib.la_segments.restype = ctypes.c_int
    lib.la_strerror.argtypes = [i]
    lib.la_strerror.restype = ctypes.c_char_p
    lib.la_version.argtypes = []
    lib.la_version.restype = ctypes.c_int
    return lib


def hip_runtimes() -> list:
    """Paths of the HIP runtime libraries (libamdhip64) mapped into this process."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 6 and "libamdhip64" in parts[-1]:
                paths.add(os.path.realpath(parts[-1]))
    return sorted(paths)


lib = _load(LIB_PATH)
if len(hip_runtimes()) > 1:
    # two runtimes in one process do not share devices, memory or streams: the library's calls
    # on PyTorch's tensors would fault, so refuse here instead
    raise ImportError("liblinattn bound to a second HIP runtime (import torch before this "
                      f"package): {hip_runtimes()}")


def strerror(status: int) -> str:
    return lib.la_strerror(int(status)).decode()


def version() -> tuple:
    v = lib.la_version()
    return (v >> 16, (v >> 8) & 0xFF, v & 0xFF)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return LA_BF16
    if t.dtype == torch.float32:
        return LA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    # (ctypes takes a plain int for a void * argument)
    return None if t is None else t.data_ptr()


# the raw handle of a device's current stream: torch's own accessor where it has one (no Stream
# object per call: a few microseconds of host time on small calls), else the public one
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t):
    if _raw_stream is not None:
        return _raw_stream(t.device.index)
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_tensors(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("liblinattn takes device tensors only")
        if not t.is_contiguous():
            raise ValueError("liblinattn takes contiguous tensors only")
        if dev is not None and t.device != dev:
            raise ValueError("all tensors must be on one device")
        dev = t.device


def _dims(q, k, v):
    if k.dim() == 3:  # decode tensors given as [B, H, d]
        B, H, d = k.shape
        return B, H, 1, d, v.shape[-1]
    if k.dim() != 4 or v.dim() != 4:
        raise ValueError(f"k and v must be [B, H, N, d] tensors, got {tuple(k.shape)} and "
                         f"{tuple(v.shape)}")
    B, H, N, d = k.shape
    return B, H, N, d, v.shape[-1]


def _expect(name, t, shape, dtype):
    """Raises ValueError unless tensor t (if given) has exactly this shape and dtype: the C ABI
    sees only pointers and sizes, so a mismatched buffer would be read or written past its
    end."""
    if t is None:
        return
    if t.shape != shape:
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _layout(q, k, v, out, states=(), rows=None):
    """Checks q, k [B,H,N,d], v, out [B,H,N,d_v] (decode: N = 1 given as [B,H,d] and
    [B,H,d_v], or [B,H,1,.]) of one input dtype, and each float32 state pair (S, z) in
    ``states`` against [B,H,rows,d_v] and [B,H,rows] (rows = d unless given). Returns
    (B, H, N, d, d_v) as k and v give them."""
    B, H, N, d, dv = _dims(q, k, v)
    dt = k.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise TypeError(f"unsupported dtype {dt}")
    lead = tuple(k.shape[:-1])
    _expect("v", v, lead + (dv,), dt)
    _expect("q", q, tuple(k.shape), dt)
    _expect("out", out, lead + (dv,), dt)
    r = d if rows is None else rows
    for S, z in states:
        _expect("S", S, (B, H, r, dv), torch.float32)
        _expect("z", z, (B, H, r), torch.float32)
    return B, H, N, d, dv


def _check(status, fn):
    if status != LA_OK:
        raise LAError(status, fn)


def la_causal_fwd(q, k, v, out, S=None, z=None, chunk: int = 0, seg_len: int = 0):
    """Causal prefill (see include/la.h). S, z: optional float32 in/out state."""
    B, H, N, d, dv = _layout(q, k, v, out, states=((S, z),))
    _check_tensors(q, k, v, out, S, z)
    st = lib.la_causal_fwd_seg(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S), _ptr(z), B, H, N, d,
                               dv, chunk, seg_len, _dtype_code(k), _stream(k))
    _check(st, "la_causal_fwd")
    return out


def la_causal_fwd_state(q, k, v, out, S0=None, z0=None, S=None, z=None, chunk: int = 0,
                        seg_len: int = 0):
    """Causal prefill with the initial state (S0, z0; None: zero) and the final state (S, z;
    None: not returned) in separate float32 tensors (see include/la.h)."""
    B, H, N, d, dv = _layout(q, k, v, out, states=((S0, z0), (S, z)))
    _check_tensors(q, k, v, out, S0, z0, S, z)
    st = lib.la_causal_fwd_state(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S0), _ptr(z0), _ptr(S),
                                 _ptr(z), B, H, N, d, dv, chunk, seg_len, _dtype_code(k), _stream(k))
    _check(st, "la_causal_fwd_state")
    return out


def la_causal_fwd_ex(q, k, v, out, S0=None, z0=None, S=None, z=None, chunk: int = 0,
                     seg_len: int = 0, flags: int = 0):
    """la_causal_fwd_state with variant flags (LA_PHI_IDENTITY, LA_UNNORMALIZED)."""
    B, H, N, d, dv = _layout(q, k, v, out, states=((S0, z0), (S, z)))
    _check_tensors(q, k, v, out, S0, z0, S, z)
    st = lib.la_causal_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S0), _ptr(z0), _ptr(S),
                              _ptr(z), B, H, N, d, dv, chunk, seg_len, flags, _dtype_code(k),
                              _stream(k))
    _check(st, "la_causal_fwd_ex")
    return out


def la_causal_fwd_profiled(q, k, v, out, S0=None, z0=None, S=None, z=None, chunk: int = 0,
                           seg_len: int = 0, flags: int = 0, reps: int = 1):
    """la_causal_fwd_ex enqueued `reps` times back to back with HIP events around its
    kernels; waits for them and returns the average device milliseconds of (segment sums,
    segment scan, causal outputs)."""
    B, H, N, d, dv = _layout(q, k, v, out, states=((S0, z0), (S, z)))
    _check_tensors(q, k, v, out, S0, z0, S, z)
    ms = (ctypes.c_float * 3)()
    st = lib.la_causal_fwd_profiled(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S0), _ptr(z0),
                                    _ptr(S), _ptr(z), B, H, N, d, dv, chunk, seg_len, flags,
                                    _dtype_code(k), _stream(k), reps, ms)
    _check(st, "la_causal_fwd_profiled")
    return tuple(float(x) for x in ms)


def la_global_fwd(q, k, v, out, S, z, chunk: int = 0):
    """Global (non-causal) form; S, z are written. q and out may both be None."""
    B, H, N, d, dv = _layout(q, k, v, out, states=((S, z),))
    _check_tensors(q, k, v, out, S, z)
    st = lib.la_global_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S), _ptr(z), B, H, N, d, dv,
                           chunk, _dtype_code(k), _stream(k))
    _check(st, "la_global_fwd")
    return out


def la_global_fwd_ex(q, k, v, out, S, z, chunk: int = 0, flags: int = 0):
    """la_global_fwd with variant flags."""
    B, H, N, d, dv = _layout(q, k, v, out, states=((S, z),))
    _check_tensors(q, k, v, out, S, z)
    st = lib.la_global_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S), _ptr(z), B, H, N, d,
                              dv, chunk, flags, _dtype_code(k), _stream(k))
    _check(st, "la_global_fwd_ex")
    return out


def la_decode_step(q, k, v, out, S, z):
    """One decode step; S, z are updated in place."""
    B, H, N, d, dv = _layout(q, k, v, out, states=((S, z),))
    _check_tensors(q, k, v, out, S, z)
    st = lib.la_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S), _ptr(z), B, H, N, d, dv,
                            0, _dtype_code(k), _stream(k))
    _check(st, "la_decode_step")
    return out


def la_decode_step_ex(q, k, v, out, S, z, flags: int = 0):
    """la_decode_step with variant flags."""
    B, H, N, d, dv = _layout(q, k, v, out, states=((S, z),))
    _check_tensors(q, k, v, out, S, z)
    st = lib.la_decode_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S), _ptr(z), B, H, N, d,
                               dv, flags, _dtype_code(k), _stream(k))
    _check(st, "la_decode_step_ex")
    return out


def la_causal_fwd_decay(q, k, v, out, gamma, S0=None, z0=None, S=None, z=None, chunk: int = 0,
                        seg_len: int = 0, flags: int = 0):
    """Causal prefill of the decayed recurrence; gamma: float32 [H] on the device."""
    B, H, N, d, dv = _layout(q, k, v, out, states=((S0, z0), (S, z)))
    if gamma is None or gamma.dtype != torch.float32 or gamma.numel() != H:
        raise ValueError("gamma must be a float32 tensor of H values")
    _check_tensors(q, k, v, out, gamma, S0, z0, S, z)
    st = lib.la_causal_fwd_decay(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S0), _ptr(z0), _ptr(S),
                                 _ptr(z), _ptr(gamma), B, H, N, d, dv, chunk, seg_len, flags,
                                 _dtype_code(k), _stream(k))
    _check(st, "la_causal_fwd_decay")
    return out


def la_decode_step_decay(q, k, v, out, S, z, gamma, flags: int = 0):
    """One decode step of the decayed recurrence; S, z are updated in place."""
    B, H, N, d, dv = _layout(q, k, v, out, states=((S, z),))
    if gamma is None or gamma.dtype != torch.float32 or gamma.numel() != H:
        raise ValueError("gamma must be a float32 tensor of H values")
    _check_tensors(q, k, v, out, S, z, gamma)
    st = lib.la_decode_step_decay(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S), _ptr(z),
                                  _ptr(gamma), B, H, N, d, dv, flags, _dtype_code(k), _stream(k))
    _check(st, "la_decode_step_decay")
    return out


def _workspace(ws, need):
    """ws: a device tensor of at least `need` bytes (contiguous), or None when need is 0."""
    if ws is None:
        if need:
            raise ValueError(f"this call needs a workspace of {need} bytes")
        return None, 0
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise ValueError(f"workspace holds {nbytes} bytes, the call needs {need}")
    return ws, nbytes


def la_causal_fwd_ws(q, k, v, out, ws, S0=None, z0=None, S=None, z=None, gamma=None,
                     chunk: int = 0, seg_len: int = 0, flags: int = 0):
    """Causal prefill with a caller-supplied workspace `ws` (a device tensor of at least
    la_workspace_bytes(0, ...) bytes; None when that is 0): la_causal_fwd_ex, or
    la_causal_fwd_decay when gamma is given. Allocates nothing and never waits."""
    B, H, N, d, dv = _layout(q, k, v, out, states=((S0, z0), (S, z)))
    if gamma is not None and (gamma.dtype != torch.float32 or gamma.numel() != H):
        raise ValueError("gamma must be a float32 tensor of H values")
    need = la_workspace_bytes(0, B, H, N, d, dv, chunk, seg_len, _dtype_code(k))
    ws, nbytes = _workspace(ws, need)
    _check_tensors(q, k, v, out, S0, z0, S, z, gamma, ws)
    st = lib.la_causal_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S0), _ptr(z0), _ptr(S),
                              _ptr(z), _ptr(gamma), B, H, N, d, dv, chunk, seg_len, flags,
                              _dtype_code(k), _ptr(ws), nbytes, _stream(k))
    _check(st, "la_causal_fwd_ws")
    return out


def la_global_fwd_ws(q, k, v, out, S, z, ws, chunk: int = 0, flags: int = 0):
    """Global form with a caller-supplied workspace `ws` (at least la_workspace_bytes(1, ...)
    bytes; None when that is 0). q and out may both be None."""
    B, H, N, d, dv = _layout(q, k, v, out, states=((S, z),))
    need = la_workspace_bytes(1, B, H, N, d, dv, chunk, 0, _dtype_code(k))
    ws, nbytes = _workspace(ws, need)
    _check_tensors(q, k, v, out, S, z, ws)
    st = lib.la_global_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S), _ptr(z), B, H, N, d,
                              dv, chunk, flags, _dtype_code(k), _ptr(ws), nbytes, _stream(k))
    _check(st, "la_global_fwd_ws")
    return out


def la_causal_fwd_noalloc(q, k, v, out, S0=None, z0=None, S=None, z=None, chunk: int = 0,
                          seg_len: int = 0, flags: int = 0):
    """la_causal_fwd_ex with the segment states in the library's static per-device scratch
    array (64 MiB): allocates nothing. Calls that overlap in time on one device race."""
    B, H, N, d, dv = _layout(q, k, v, out, states=((S0, z0), (S, z)))
    _check_tensors(q, k, v, out, S0, z0, S, z)
    st = lib.la_causal_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S0), _ptr(z0),
                                   _ptr(S), _ptr(z), B, H, N, d, dv, chunk, seg_len, flags,
                                   _dtype_code(k), _stream(k))
    _check(st, "la_causal_fwd_noalloc")
    return out


def la_release_cache():
    """Frees the scratch blocks the convenience entry points cached (waits for their last use)."""
    _check(lib.la_release_cache(), "la_release_cache")


def la_causal_fwd_rf(q, k, v, out, W, S0=None, z0=None, S=None, z=None, chunk: int = 0,
                     seg_len: int = 0, flags: int = 0):
    """Causal prefill over positive random features of q and k (projections W [m, d]); the
    state S [B,H,m,d_v], z [B,H,m] as for la_causal_fwd_state."""
    if W is None or W.dim() != 2:
        raise ValueError("W must be a [m, d] tensor")
    m = W.shape[0]
    B, H, N, d, dv = _layout(q, k, v, out, states=((S0, z0), (S, z)), rows=m)
    _expect("W", W, (m, d), k.dtype)
    _check_tensors(q, k, v, out, W, S0, z0, S, z)
    st = lib.la_causal_fwd_rf(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(W), _ptr(S0), _ptr(z0),
                              _ptr(S), _ptr(z), B, H, N, d, dv, m, chunk, seg_len, flags,
                              _dtype_code(k), _stream(k))
    _check(st, "la_causal_fwd_rf")
    return out


def la_rf_features(x, W, f):
    """Positive random features f[..., r] = exp(W[r] . x - |x|^2 / 2) / sqrt(m) of the rows of
    x [..., d] for projections W [m, d]; f [..., m] (all one dtype, contiguous, on the GPU)."""
    if W.dim() != 2:
        raise ValueError("W must be a [m, d] tensor")
    m, d = W.shape
    if x.shape[-1] != d or f.shape[-1] != m or x.shape[:-1] != f.shape[:-1]:
        raise ValueError(f"shapes x {tuple(x.shape)}, W {tuple(W.shape)}, f {tuple(f.shape)} do not match")
    if x.dtype != W.dtype or x.dtype != f.dtype:
        raise ValueError("x, W and f must share one dtype")
    _check_tensors(x, W, f)
    rows = x.numel() // d if d else 0
    st = lib.la_rf_features(_ptr(x), _ptr(W), _ptr(f), rows, d, m, _dtype_code(x), _stream(x))
    _check(st, "la_rf_features")
    return f


def la_segments(form: int, B: int, H: int, N: int, d: int, d_v: int, chunk: int = 0,
                seg_len: int = 0, dtype: int = LA_BF16) -> int:
    return int(lib.la_segments(form, B, H, N, d, d_v, chunk, seg_len, dtype))


@functools.lru_cache(maxsize=1024)
def la_workspace_bytes(form: int, B: int, H: int, N: int, d: int, d_v: int, chunk: int = 0,
                       seg_len: int = 0, dtype: int = LA_BF16) -> int:
    # a function of its arguments alone, so it is asked of the library once per shape
    return int(lib.la_workspace_bytes(form, B, H, N, d, d_v, chunk, seg_len, dtype))
