"""MI355X (gfx950) k-means assignment and centroid update: Python binding of
``libkmeans_mi355x.so``.

The functions here only marshal torch tensors into the C ABI declared in
``include/kmeans_mi355x.h`` (device pointers, sizes, the current HIP stream);
every step of the computation runs in the library's HIP kernels.  There is no
CPU fallback: if the library is missing, the first call raises.

    norms = kmeans_centroid_norms(C)                    # fp32 [K]
    labels, min_dist = kmeans_assign(X, C, norms)       # int32 [N], fp32 [N]
    C, norms, counts, _ = kmeans_update(X, labels, C)   # next Lloyd iterate

``X`` and ``C`` are ``torch.bfloat16`` CUDA tensors of shape ``[N, D]`` and
``[K, D]``, contiguous.  Calls are asynchronous on the current stream.
"""

from __future__ import annotations

import contextlib
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# The built library; KMEANS_MI355X_LIBRARY names another build of the same
# sources instead (the host-sanitizer test loads one built with AddressSanitizer).
LIBRARY = os.environ.get("KMEANS_MI355X_LIBRARY") or os.path.join(_HERE, "libkmeans_mi355x.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "kmeans_mi355x.h")

KMEANS_OK = 0
KMEANS_ERR_INVALID_ARG = 1
KMEANS_ERR_UNSUPPORTED = 2
KMEANS_ERR_ALIGNMENT = 3
KMEANS_ERR_HIP = 4
KMEANS_ERR_NO_MEMORY = 5

PATH_AUTO = 0
PATH_DIRECT = 1
PATH_SPLIT = 2
PATH_PERSISTENT = 3
# kmeans_update_path_t
UPDATE_AUTO = 0
UPDATE_SORT = 1
UPDATE_BUCKETS = 2

_STATUS_NAMES = {
    0: "KMEANS_OK", 1: "KMEANS_ERR_INVALID_ARG", 2: "KMEANS_ERR_UNSUPPORTED",
    3: "KMEANS_ERR_ALIGNMENT", 4: "KMEANS_ERR_HIP", 5: "KMEANS_ERR_NO_MEMORY",
}

_lib = None


class KmeansError(RuntimeError):
    """A non-OK status from the C ABI."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load_library(path: str = LIBRARY):
    """Load the HIP library (after torch, so both use one HIP runtime)."""
    global _lib
    if _lib is not None and path == LIBRARY:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library {path} is not built; run `python -m "
            "means_nearest_centroid_amd.build` (or __graft_entry__.build())")
    try:
        import torch  # noqa: F401  -- maps torch's libamdhip64 first
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.kmeans_centroid_norms.argtypes = [vp, i64, i64, vp, vp]
    lib.kmeans_centroid_norms.restype = ctypes.c_int
    lib.kmeans_assign.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, vp]
    lib.kmeans_assign.restype = ctypes.c_int
    lib.kmeans_assign_static.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, vp]
    lib.kmeans_assign_static.restype = ctypes.c_int
    lib.kmeans_assign_path.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i32, i32, vp]
    lib.kmeans_assign_path.restype = ctypes.c_int
    lib.kmeans_plan.argtypes = [i64, i64, i64, i32, i32p, i32p, i32p, i32p, i32p, i32p]
    lib.kmeans_plan.restype = ctypes.c_int
    lib.kmeans_update.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, vp, vp, vp]
    lib.kmeans_update.restype = ctypes.c_int
    lib.kmeans_update_path.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, vp, vp, i32, vp]
    lib.kmeans_update_path.restype = ctypes.c_int
    lib.kmeans_release_workspace.argtypes = [vp]
    lib.kmeans_release_workspace.restype = ctypes.c_int
    lib.kmeans_last_error.argtypes = []
    lib.kmeans_last_error.restype = ctypes.c_char_p
    lib.kmeans_abi_version.argtypes = []
    lib.kmeans_abi_version.restype = ctypes.c_int
    if path == LIBRARY:
        _lib = lib
    return lib


def _check(lib, status: int):
    if status != KMEANS_OK:
        raise KmeansError(status, lib.kmeans_last_error().decode(errors="replace"))


def _stream_handle(stream, device=None):
    """The HIP stream to launch on, as an integer handle: ``stream``, or the
    current stream of ``device`` (of the current device when None).  Calls
    are often a few microseconds of GPU time, so this avoids building a
    torch Stream object per call where torch exposes the raw handle."""
    import torch
    if stream is None:
        index = device.index if device is not None else torch.cuda.current_device()
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return raw(index)
        return torch.cuda.current_stream(index).cuda_stream
    if device is not None and stream.device != device:
        raise ValueError(f"stream is on {stream.device} but the tensors on {device}")
    return stream.cuda_stream


def _on(device):
    """The library launches on the current HIP device: make it the tensors'
    (a no-op context when it already is)."""
    import torch
    if device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def _ptr(t):
    return t.data_ptr() if t is not None else None


def _matrix(t, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16 or t.dim() != 2 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 2-D torch.bfloat16 CUDA tensor "
                         f"(got {t.dtype}, {tuple(t.shape)}, {t.device})")
    return t


def _vector(t, name, dtype, n, device):
    """Check a caller-supplied 1-D output (or input) tensor: the C ABI sees
    only a pointer, so a wrong dtype, a short tensor or a strided view would
    be written out of bounds without an error."""
    import torch
    if (not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda
            or t.device != device or t.numel() != n or not t.is_contiguous()):
        got = (f"{t.dtype}, {tuple(t.shape)}, {t.device}, contiguous={t.is_contiguous()}"
               if isinstance(t, torch.Tensor) else type(t).__name__)
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of {n} elements "
                         f"on {device} (got {got})")
    return t


def abi_version() -> int:
    return load_library().kmeans_abi_version()


def kmeans_plan(N: int, D: int, K: int, compute_units: int = 0) -> dict:
    """Launch plan the library would use for a shape on a GPU with
    ``compute_units`` CUs (0: 256, an MI355X); no GPU needed."""
    lib = load_library()
    vals = [ctypes.c_int32(0) for _ in range(6)]
    _check(lib, lib.kmeans_plan(N, D, K, compute_units, *[ctypes.byref(v) for v in vals]))
    keys = ("path", "splits", "workgroups", "points_per_wg", "k_block", "padded_d")
    return {k: v.value for k, v in zip(keys, vals)}


def kmeans_centroid_norms(C, norms=None, stream=None):
    """``norms[k] = sum_j C[k, j]**2`` (fp32), asynchronously on ``stream``."""
    import torch
    C = _matrix(C, "C")
    K, D = C.shape
    if norms is None:
        norms = torch.empty(K, dtype=torch.float32, device=C.device)
    _vector(norms, "norms", torch.float32, K, C.device)
    lib = load_library()
    with _on(C.device):
        _check(lib, lib.kmeans_centroid_norms(_ptr(C), K, D, _ptr(norms),
                                              _stream_handle(stream, C.device)))
    return norms


def _assign_args(X, C, norms, labels, min_dist):
    import torch
    X = _matrix(X, "X")
    C = _matrix(C, "C")
    N, D = X.shape
    K = C.shape[0]
    if C.shape[1] != D:
        raise ValueError(f"X has D={D} but C has D={C.shape[1]}")
    if C.device != X.device:
        raise ValueError(f"X is on {X.device} but C on {C.device}")
    _vector(norms, "norms", torch.float32, K, X.device)
    if labels is None:
        labels = torch.empty(N, dtype=torch.int32, device=X.device)
    if min_dist is None:
        min_dist = torch.empty(N, dtype=torch.float32, device=X.device)
    _vector(labels, "labels", torch.int32, N, X.device)
    _vector(min_dist, "min_dist", torch.float32, N, X.device)
    return X, C, norms, N, D, K, labels, min_dist


def kmeans_assign(X, C, norms, labels=None, min_dist=None, stream=None):
    """Nearest centroid per point: ``(labels int32 [N], min_dist fp32 [N])``."""
    X, C, norms, N, D, K, labels, min_dist = _assign_args(X, C, norms, labels, min_dist)
    lib = load_library()
    with _on(X.device):
        _check(lib, lib.kmeans_assign(_ptr(X), _ptr(C), _ptr(norms), N, D, K, _ptr(labels),
                                      _ptr(min_dist), _stream_handle(stream, X.device)))
    return labels, min_dist


def kmeans_assign_static(X, C, norms, labels=None, min_dist=None, stream=None):
    """``kmeans_assign`` whose K-split scratch is the library's fixed device
    buffer (no allocation inside the call; give ``labels`` and ``min_dist``
    to allocate nothing at all).  Calls that overlap on one GPU race."""
    X, C, norms, N, D, K, labels, min_dist = _assign_args(X, C, norms, labels, min_dist)
    lib = load_library()
    with _on(X.device):
        _check(lib, lib.kmeans_assign_static(_ptr(X), _ptr(C), _ptr(norms), N, D, K,
                                             _ptr(labels), _ptr(min_dist),
                                             _stream_handle(stream, X.device)))
    return labels, min_dist


def kmeans_assign_path(X, C, norms, path: int = PATH_AUTO, count: int = 0,
                       labels=None, min_dist=None, stream=None):
    """``kmeans_assign`` with a forced path (``PATH_DIRECT``, ``PATH_SPLIT`` or
    ``PATH_PERSISTENT``).  ``count``: for the split path the number of
    K-ranges (0: automatic); for the direct path 1 selects narrow point tiles
    (32 points per wave), any other value wide ones; for the persistent path
    the number of workgroups (0: one per CU)."""
    X, C, norms, N, D, K, labels, min_dist = _assign_args(X, C, norms, labels, min_dist)
    lib = load_library()
    with _on(X.device):
        _check(lib, lib.kmeans_assign_path(_ptr(X), _ptr(C), _ptr(norms), N, D, K,
                                           _ptr(labels), _ptr(min_dist), path, count,
                                           _stream_handle(stream, X.device)))
    return labels, min_dist


def kmeans_update(X, labels, C_old, C_new=None, norms=None, counts=None, means=None,
                  with_means: bool = False, stream=None, path: int = UPDATE_AUTO):
    """Centroid update from ``labels``: ``(C_new bf16 [K, D], norms fp32 [K],
    counts int32 [K], means fp32 [K, D] or None)``.  An empty cluster keeps
    its row of ``C_old``; labels outside ``[0, K)`` count for no cluster.
    ``C_new`` may be ``C_old`` itself (in-place update).  ``path``:
    ``UPDATE_AUTO``, ``UPDATE_SORT`` or ``UPDATE_BUCKETS`` (kmeans_update_path)."""
    import torch
    X = _matrix(X, "X")
    C_old = _matrix(C_old, "C_old")
    N, D = X.shape
    K = C_old.shape[0]
    if C_old.shape[1] != D:
        raise ValueError(f"X has D={D} but C_old has D={C_old.shape[1]}")
    if C_old.device != X.device:
        raise ValueError(f"X is on {X.device} but C_old on {C_old.device}")
    dev = C_old.device
    _vector(labels, "labels", torch.int32, N, dev)
    if C_new is None:
        C_new = torch.empty_like(C_old)
    else:
        C_new = _matrix(C_new, "C_new")
        if C_new.shape != C_old.shape:
            raise ValueError("C_new must have the shape of C_old")
    if norms is None:
        norms = torch.empty(K, dtype=torch.float32, device=dev)
    if counts is None:
        counts = torch.empty(K, dtype=torch.int32, device=dev)
    if means is None and with_means:
        means = torch.empty((K, D), dtype=torch.float32, device=dev)
    if C_new.device != dev:
        raise ValueError(f"C_new must be on {dev}")
    for t, name, dt, n in ((norms, "norms", torch.float32, K), (counts, "counts", torch.int32, K),
                           (means, "means", torch.float32, K * D)):
        if t is not None:
            _vector(t, name, dt, n, dev)
    lib = load_library()
    with _on(dev):
        _check(lib, lib.kmeans_update_path(_ptr(X), _ptr(labels), _ptr(C_old), N, D, K,
                                           _ptr(C_new), _ptr(norms), _ptr(counts), _ptr(means),
                                           int(path), _stream_handle(stream, dev)))
    return C_new, norms, counts, means


def kmeans_release_workspace(stream=None):
    """Return the stream's workspace (the K-split path's and the update's
    scratch, kept between calls) and its tile queue (the persistent path's)
    to the device's memory pool, in stream order; a later call on the stream
    allocates them again."""
    lib = load_library()
    _check(lib, lib.kmeans_release_workspace(_stream_handle(stream)))


def assign(X, C, norms=None):
    """Convenience: compute the norms if not given, then assign."""
    if norms is None:
        norms = kmeans_centroid_norms(C)
    return kmeans_assign(X, C, norms)
