"""Thin ctypes binding of libflashhead (argument marshalling only).

Every step of the head runs in the library's HIP kernels.  PyTorch is used
for device memory and streams: tensors are passed as raw device pointers and
the current torch stream as the hipStream_t.  If the library is missing the
import of this module fails loudly; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# FLASHHEAD_LIB_VARIANT=trace loads the measurement build (timeline hooks)
_VARIANT = os.environ.get("FLASHHEAD_LIB_VARIANT", "")
if _VARIANT not in ("", "trace"):
    raise ImportError(f"unknown FLASHHEAD_LIB_VARIANT {_VARIANT!r}")
LIB_PATH = os.path.join(_PKG, "libflashhead_trace.so" if _VARIANT else "libflashhead.so")

FH_OK = 0
FH_ERR_INVALID_ARG = -1
FH_ERR_NOT_PERMUTATION = -2
FH_ERR_UNSUPPORTED = -3
FH_ERR_HIP = -4
FH_ERR_OOM = -5
FH_DTYPE_F32 = 0
FH_DTYPE_BF16 = 1
FH_QUANT_NONE = 0
FH_QUANT_INT4_G128 = 1
FH_QUANT_INT4_G128_MEAN = 2
FH_MODE_GREEDY = 0
FH_MODE_SAMPLE = 1
FH_FLAG_COOPERATIVE = 1
FH_FLAG_BORROW_E = 2
FH_FLAG_STREAM_ALL = 4
FH_FLAG_SELECT_FIRST = 8

EXPORTED = [
    "flashhead_prepare", "flashhead_destroy", "flashhead_greedy",
    "flashhead_sample", "dense_head_workspace_bytes", "dense_head",
    "flashhead_status_string", "flashhead_export_centroids",
    "flashhead_export_int4", "flashhead_query", "flashhead_profile_begin",
    "flashhead_profile_end", "flashhead_last_hip_error", "flashhead_stream_read",
    "flashhead_mc_workspace_bytes", "flashhead_mc_marginal", "flashhead_kmeans",
    "flashhead_plan_step", "dense_head_static", "flashhead_trace_read",
    "flashhead_greedy_adaptive", "flashhead_sample_adaptive",
]
FH_DENSE_STATIC_MAX_BATCH = 16


class fh_desc(C.Structure):
    _fields_ = [("v", C.c_int64), ("d", C.c_int32), ("c", C.c_int32),
                ("b", C.c_int32), ("dtype", C.c_int32), ("lde", C.c_int64),
                ("E", C.c_void_p), ("c2t", C.c_void_p), ("C", C.c_void_p),
                ("quant", C.c_int32), ("max_batch", C.c_int32),
                ("max_p", C.c_int32), ("stream", C.c_void_p),
                ("flags", C.c_int32)]


class fh_debug(C.Structure):
    _fields_ = [("scores", C.c_void_p), ("clusters", C.c_void_p),
                ("cand_ids", C.c_void_p), ("cand_logits", C.c_void_p)]


class FlashHeadError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = f"{what}: {status_string(status)} ({status})"
        if status in (FH_ERR_HIP, FH_ERR_OOM):
            msg += f" [{flashhead_last_hip_error()}]"
        super().__init__(msg)
        self.status = status


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first "
            "(python -m two_stage_retrieval_amd.build)")
    lib = C.CDLL(LIB_PATH)
    vp, i32, i64, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_float
    lib.flashhead_prepare.argtypes = [C.POINTER(fh_desc), C.POINTER(vp)]
    lib.flashhead_prepare.restype = C.c_int
    lib.flashhead_destroy.argtypes = [vp]
    lib.flashhead_destroy.restype = None
    lib.flashhead_greedy.argtypes = [vp, vp, i32, i32, vp,
                                     C.POINTER(fh_debug), vp]
    lib.flashhead_greedy.restype = C.c_int
    lib.flashhead_sample.argtypes = [vp, vp, i32, i32, f32, vp, vp, vp,
                                     C.POINTER(fh_debug), vp]
    lib.flashhead_sample.restype = C.c_int
    lib.flashhead_greedy_adaptive.argtypes = [vp, vp, i32, i32, i32, f32, vp, vp,
                                              C.POINTER(fh_debug), vp]
    lib.flashhead_greedy_adaptive.restype = C.c_int
    lib.flashhead_sample_adaptive.argtypes = [vp, vp, i32, i32, i32, f32, f32, vp, vp, vp,
                                              vp, C.POINTER(fh_debug), vp]
    lib.flashhead_sample_adaptive.restype = C.c_int
    lib.dense_head_workspace_bytes.argtypes = [i32]
    lib.dense_head_workspace_bytes.restype = C.c_size_t
    lib.dense_head.argtypes = [vp, i64, i32, i32, i64, vp, i32, i32, f32, vp,
                               vp, vp, vp, vp]
    lib.dense_head.restype = C.c_int
    lib.dense_head_static.argtypes = [vp, i64, i32, i32, i64, vp, i32, i32, f32, vp,
                                      vp, vp, vp]
    lib.dense_head_static.restype = C.c_int
    lib.flashhead_status_string.argtypes = [C.c_int]
    lib.flashhead_status_string.restype = C.c_char_p
    lib.flashhead_stream_read.argtypes = [vp, i64, vp, vp]
    lib.flashhead_stream_read.restype = C.c_int
    lib.flashhead_last_hip_error.argtypes = []
    lib.flashhead_last_hip_error.restype = C.c_char_p
    lib.flashhead_export_centroids.argtypes = [vp, vp]
    lib.flashhead_export_centroids.restype = C.c_int
    lib.flashhead_export_int4.argtypes = [vp, vp, vp]
    lib.flashhead_export_int4.restype = C.c_int
    lib.flashhead_query.argtypes = [vp, i32, C.POINTER(i64)]
    lib.flashhead_query.restype = C.c_int
    lib.flashhead_profile_begin.argtypes = [vp, i32]
    lib.flashhead_profile_begin.restype = C.c_int
    lib.flashhead_profile_end.argtypes = [vp, C.POINTER(C.c_double),
                                          C.POINTER(i32)]
    lib.flashhead_profile_end.restype = C.c_int
    lib.flashhead_mc_workspace_bytes.argtypes = [vp, i32, i32, i32]
    lib.flashhead_mc_workspace_bytes.restype = C.c_size_t
    lib.flashhead_mc_marginal.argtypes = [vp, vp, i32, f32, vp, i32, vp, i32,
                                          vp, vp, vp, C.c_size_t, vp]
    lib.flashhead_mc_marginal.restype = C.c_int
    lib.flashhead_kmeans.argtypes = [vp, i64, i32, i32, i64, i32, vp, i32, vp, vp,
                                     C.POINTER(i32), vp]
    lib.flashhead_kmeans.restype = C.c_int
    lib.flashhead_plan_step.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                        C.POINTER(i32)]
    lib.flashhead_plan_step.restype = C.c_int
    lib.flashhead_trace_read.argtypes = [vp, i64, C.POINTER(i64), C.POINTER(i64)]
    lib.flashhead_trace_read.restype = C.c_int
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.flashhead_status_string(status).decode()


def flashhead_stream_read(buf, sink, stream=None) -> None:
    """Streaming read of a whole device tensor (measurement reference)."""
    _check(lib.flashhead_stream_read(_ptr(buf), buf.numel() * buf.element_size(),
                                     _ptr(sink), _stream(stream)), "flashhead_stream_read")


def flashhead_last_hip_error() -> str:
    return lib.flashhead_last_hip_error().decode()


def _check(status: int, what: str) -> None:
    if status != FH_OK:
        raise FlashHeadError(status, what)


# --------------------------------------------------------------------------
# marshalling helpers (torch is imported lazily: host-only users need none)
# --------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    if stream is not None:
        return stream
    torch = _torch()
    return torch.cuda.current_stream().cuda_stream


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return FH_DTYPE_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return FH_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _debug(dbg: Optional[dict]):
    if not dbg:
        return None
    d = fh_debug(_ptr(dbg.get("scores")), _ptr(dbg.get("clusters")),
                 _ptr(dbg.get("cand_ids")), _ptr(dbg.get("cand_logits")))
    return C.byref(d), d


# --------------------------------------------------------------------------
# the C calls under their own names
# --------------------------------------------------------------------------

def flashhead_prepare(E, c2t: np.ndarray, C_init=None, *, v=None, d=None,
                      lde=None, quant: int = FH_QUANT_NONE, max_batch: int = 1,
                      max_p: int = 1, flags: int = 0, stream=None) -> int:
    """Returns an opaque handle (int).  E, C_init: device tensors."""
    c2t = np.ascontiguousarray(c2t, dtype=np.int32)
    c, b = c2t.shape
    v = v if v is not None else E.shape[0]
    d = d if d is not None else E.shape[1]
    lde = lde if lde is not None else E.stride(0)
    desc = fh_desc(v, d, c, b, dtype_code(E), lde, _ptr(E),
                   c2t.ctypes.data, _ptr(C_init), quant, max_batch, max_p,
                   _stream(stream), flags)
    h = C.c_void_p()
    _check(lib.flashhead_prepare(C.byref(desc), C.byref(h)),
           "flashhead_prepare")
    return h.value


def flashhead_plan_step(c: int, b: int, d: int, dtype: int, quant: int, B: int,
                        p: int, num_cu: int, blocks_per_cu: int, flags: int = 0):
    """Host-only: (path, grid) a decode step of this shape takes."""
    g = C.c_int32()
    st = lib.flashhead_plan_step(c, b, d, dtype, quant, B, p, num_cu, blocks_per_cu, flags,
                                 C.byref(g))
    if st < 0:
        raise FlashHeadError(st, "flashhead_plan_step")
    return st, g.value


def flashhead_trace_read():
    """(words as a numpy uint64 array, device clock kHz) from the
    measurement build; FlashHeadError(FH_ERR_UNSUPPORTED) from the library."""
    n, khz = C.c_int64(), C.c_int64()
    buf = np.zeros(1 << 16, dtype=np.uint64)
    _check(lib.flashhead_trace_read(buf.ctypes.data, buf.size, C.byref(n), C.byref(khz)),
           "flashhead_trace_read")
    return buf[:n.value].copy(), khz.value


def flashhead_destroy(handle: int) -> None:
    lib.flashhead_destroy(handle)


def flashhead_greedy(handle: int, H, B: int, p: int, out_tokens,
                     debug: Optional[dict] = None, stream=None) -> None:
    dbg = _debug(debug)
    _check(lib.flashhead_greedy(handle, _ptr(H), B, p, _ptr(out_tokens),
                                dbg[0] if dbg else None, _stream(stream)),
           "flashhead_greedy")


def flashhead_sample(handle: int, H, B: int, p: int, tau: float, seeds,
                     out_tokens, out_lse=None, debug: Optional[dict] = None,
                     stream=None) -> None:
    dbg = _debug(debug)
    _check(lib.flashhead_sample(handle, _ptr(H), B, p, tau, _ptr(seeds),
                                _ptr(out_tokens), _ptr(out_lse),
                                dbg[0] if dbg else None, _stream(stream)),
           "flashhead_sample")


def flashhead_greedy_adaptive(handle: int, H, B: int, p_min: int, p_max: int, eps: float,
                              out_tokens, out_p=None, debug: Optional[dict] = None,
                              stream=None) -> None:
    dbg = _debug(debug)
    _check(lib.flashhead_greedy_adaptive(handle, _ptr(H), B, p_min, p_max, eps,
                                         _ptr(out_tokens), _ptr(out_p),
                                         dbg[0] if dbg else None, _stream(stream)),
           "flashhead_greedy_adaptive")


def flashhead_sample_adaptive(handle: int, H, B: int, p_min: int, p_max: int, eps: float,
                              tau: float, seeds, out_tokens, out_lse=None, out_p=None,
                              debug: Optional[dict] = None, stream=None) -> None:
    dbg = _debug(debug)
    _check(lib.flashhead_sample_adaptive(handle, _ptr(H), B, p_min, p_max, eps, tau,
                                         _ptr(seeds), _ptr(out_tokens), _ptr(out_lse),
                                         _ptr(out_p), dbg[0] if dbg else None,
                                         _stream(stream)),
           "flashhead_sample_adaptive")


def flashhead_mc_workspace_bytes(handle: int, n_draws: int, p: int,
                                 n_tokens: int) -> int:
    return int(lib.flashhead_mc_workspace_bytes(handle, n_draws, p, n_tokens))


def flashhead_mc_marginal(handle: int, H, p: int, tau: float, seeds,
                          n_draws: int, tokens, n_tokens: int, out_prob,
                          out_lse, workspace, workspace_bytes: int,
                          stream=None) -> None:
    _check(lib.flashhead_mc_marginal(handle, _ptr(H), p, tau, _ptr(seeds),
                                     n_draws, _ptr(tokens), n_tokens,
                                     _ptr(out_prob), _ptr(out_lse),
                                     _ptr(workspace), workspace_bytes,
                                     _stream(stream)),
           "flashhead_mc_marginal")


def dense_head_workspace_bytes(B: int) -> int:
    return int(lib.dense_head_workspace_bytes(B))


def dense_head(E, H, B: int, mode: int, tau: float, seeds, out_tokens,
               out_lse, workspace, *, v=None, d=None, lde=None,
               stream=None) -> None:
    v = v if v is not None else E.shape[0]
    d = d if d is not None else E.shape[1]
    lde = lde if lde is not None else E.stride(0)
    _check(lib.dense_head(_ptr(E), v, d, dtype_code(E), lde, _ptr(H), B, mode,
                          tau, _ptr(seeds), _ptr(out_tokens), _ptr(out_lse),
                          _ptr(workspace), _stream(stream)), "dense_head")


def dense_head_static(E, H, B: int, mode: int, tau: float, seeds, out_tokens,
                      out_lse=None, *, v=None, d=None, lde=None, stream=None) -> None:
    """dense_head with the library's own fixed workspace (no allocation)."""
    v = v if v is not None else E.shape[0]
    d = d if d is not None else E.shape[1]
    lde = lde if lde is not None else E.stride(0)
    _check(lib.dense_head_static(_ptr(E), v, d, dtype_code(E), lde, _ptr(H), B, mode,
                                 tau, _ptr(seeds), _ptr(out_tokens), _ptr(out_lse),
                                 _stream(stream)), "dense_head_static")


def flashhead_kmeans(E, c: int, init, max_iter: int, out_c2t, out_centroids=None, *,
                     v=None, d=None, lde=None, stream=None) -> int:
    """Equal-size spherical k-means of E's rows into c clusters (blocking).
    `init` is a host int32 array of c distinct token ids; `out_c2t` a device
    int32 tensor of c x (v / c); returns the assignments computed."""
    v = v if v is not None else E.shape[0]
    d = d if d is not None else E.shape[1]
    lde = lde if lde is not None else E.stride(0)
    init = np.ascontiguousarray(init, dtype=np.int32)
    iters = C.c_int32(0)
    _check(lib.flashhead_kmeans(_ptr(E), v, d, dtype_code(E), lde, c, init.ctypes.data,
                                max_iter, _ptr(out_c2t), _ptr(out_centroids),
                                C.byref(iters), _stream(stream)), "flashhead_kmeans")
    return int(iters.value)


def flashhead_export_centroids(handle: int, out: np.ndarray) -> np.ndarray:
    _check(lib.flashhead_export_centroids(handle, out.ctypes.data),
           "flashhead_export_centroids")
    return out


def flashhead_export_int4(handle: int, codes: np.ndarray,
                          scales: np.ndarray) -> None:
    _check(lib.flashhead_export_int4(handle, codes.ctypes.data,
                                     scales.ctypes.data),
           "flashhead_export_int4")


def flashhead_query(handle: int, what: int) -> int:
    v = C.c_int64()
    _check(lib.flashhead_query(handle, what, C.byref(v)), "flashhead_query")
    return v.value


def flashhead_profile_begin(handle: int, max_calls: int) -> None:
    _check(lib.flashhead_profile_begin(handle, max_calls),
           "flashhead_profile_begin")


def flashhead_profile_end(handle: int):
    """Returns ([stage1_ms, select_ms, stage2_ms] averages, calls)."""
    ms = (C.c_double * 3)()
    n = C.c_int32()
    _check(lib.flashhead_profile_end(handle, ms, C.byref(n)),
           "flashhead_profile_end")
    return [ms[0], ms[1], ms[2]], n.value


# --------------------------------------------------------------------------
# convenience wrapper owning a handle and its output buffers
# --------------------------------------------------------------------------

class FlashHead:
    """A prepared head on the current device (see include/flashhead.h)."""

    def __init__(self, E, c2t, C_init=None, *, quant: int = FH_QUANT_NONE,
                 max_batch: int = 1, max_p: int = 1, flags: int = 0, stream=None):
        self.E = E                      # borrowed: keep it alive
        self.c, self.b = np.asarray(c2t).shape
        self.v, self.d = E.shape
        self.quant = quant
        self.max_batch, self.max_p = max_batch, max_p
        self.handle = flashhead_prepare(E, c2t, C_init, quant=quant,
                                        max_batch=max_batch, max_p=max_p,
                                        flags=flags, stream=stream)

    def close(self):
        if getattr(self, "handle", None):
            flashhead_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def greedy(self, H, p: int, out=None, debug=None, stream=None):
        torch = _torch()
        B = H.shape[0]
        if out is None:
            out = torch.empty(B, dtype=torch.int32, device=H.device)
        flashhead_greedy(self.handle, H, B, p, out, debug, stream)
        return out

    def sample(self, H, p: int, tau: float, seeds, out=None, out_lse=None,
               debug=None, stream=None):
        torch = _torch()
        B = H.shape[0]
        if out is None:
            out = torch.empty(B, dtype=torch.int32, device=H.device)
        flashhead_sample(self.handle, H, B, p, tau, seeds, out, out_lse,
                         debug, stream)
        return out

    def greedy_adaptive(self, H, p_min: int, p_max: int, eps: float, out=None, out_p=None,
                        debug=None, stream=None):
        torch = _torch()
        B = H.shape[0]
        if out is None:
            out = torch.empty(B, dtype=torch.int32, device=H.device)
        flashhead_greedy_adaptive(self.handle, H, B, p_min, p_max, eps, out, out_p, debug,
                                  stream)
        return out

    def sample_adaptive(self, H, p_min: int, p_max: int, eps: float, tau: float, seeds,
                        out=None, out_lse=None, out_p=None, debug=None, stream=None):
        torch = _torch()
        B = H.shape[0]
        if out is None:
            out = torch.empty(B, dtype=torch.int32, device=H.device)
        flashhead_sample_adaptive(self.handle, H, B, p_min, p_max, eps, tau, seeds, out,
                                  out_lse, out_p, debug, stream)
        return out

    def mc_marginal(self, H, p: int, tau: float, seeds, tokens, out=None,
                    out_lse=None, workspace=None, stream=None):
        """Formula 7: the mean over len(seeds) draws of p(v | h, S_i) for
        each token of `tokens` (H: 1 x d)."""
        torch = _torch()
        n, q = seeds.numel(), tokens.numel()
        if out is None:
            out = torch.empty(q, dtype=torch.float32, device=H.device)
        nbytes = flashhead_mc_workspace_bytes(self.handle, n, p, q)
        if workspace is None:
            # 256-byte aligned view of a fresh byte buffer
            raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=H.device)
            off = (-raw.data_ptr()) % 256
            workspace = raw[off:off + nbytes]
        flashhead_mc_marginal(self.handle, H, p, tau, seeds, n, tokens, q, out,
                              out_lse, workspace, nbytes, stream)
        return out

    def centroids(self) -> np.ndarray:
        dt = np.float32 if self.E.element_size() == 4 else np.uint16
        out = np.empty((self.c, self.d), dtype=dt)
        return flashhead_export_centroids(self.handle, out)

    def int4(self):
        ntiles, G = (self.c + 15) // 16, self.d // 128
        codes = np.empty(ntiles * G * 1024, dtype=np.uint8)
        scales = np.empty(ntiles * G * 16, dtype=np.uint16)
        flashhead_export_int4(self.handle, codes, scales)
        return codes, scales


class DenseHead:
    """dense_head with its own zero-filled workspace."""

    def __init__(self, E, max_batch: int = 1):
        torch = _torch()
        self.E = E
        self.max_batch = max_batch
        nbytes = dense_head_workspace_bytes(max_batch)
        self.ws = torch.zeros((nbytes + 15) // 16 * 16, dtype=torch.uint8,
                              device=E.device)

    def __call__(self, H, mode=FH_MODE_GREEDY, tau=1.0, seeds=None, out=None,
                 out_lse=None, stream=None):
        torch = _torch()
        B = H.shape[0]
        if B > self.max_batch:
            raise ValueError("batch larger than the workspace")
        if out is None:
            out = torch.empty(B, dtype=torch.int32, device=H.device)
        dense_head(self.E, H, B, mode, tau, seeds, out, out_lse, self.ws,
                   stream=stream)
        return out
