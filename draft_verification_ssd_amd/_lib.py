"""ctypes binding of libssd.so: argument marshalling only; every step runs in the HIP kernels.

The functions mirror the C entry points of include/ssd.h one for one and take torch tensors
(device memory) or raw pointers. They raise RuntimeError on any non-zero status and refuse to
run when the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssd.so")
TRACE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssd_trace.so")

SSD_OK, SSD_ERR_INVALID_ARG, SSD_ERR_UNSUPPORTED, SSD_ERR_WORKSPACE, SSD_ERR_HIP, SSD_ERR_SCRATCH_LIMIT = range(6)
SSD_NOALLOC_SCRATCH_BYTES = 32 << 20
SSD_F32, SSD_BF16 = 0, 1
SSD_MAX_K, SSD_MAX_F, SSD_MAX_V, SSD_MAX_B = 16, 16, 1 << 20, 65535
SSD_DEFAULT_WAIT_POLLS = 2048


class VerifyOpts(ctypes.Structure):
    """ssd_verify_opts of include/ssd.h."""
    _fields_ = [("wait_polls", ctypes.c_int32), ("topf_last_F", ctypes.c_int32), ("topf_last_out", ctypes.c_void_p),
                ("launch_mode", ctypes.c_int32)]
FLAG_BAD_TOKEN, FLAG_SAGUARO_NORM, FLAG_BAD_F, FLAG_TIMEOUT, FLAG_BAD_C = 0x1, 0x2, 0x4, 0x8, 0x10

EXPORTS = ["ssd_verify_workspace_bytes", "ssd_verify_launches", "ssd_verify_tiles", "ssd_verify", "ssd_verify_ex",
           "ssd_stream_read", "ssd_topf_workspace_bytes",
           "ssd_topf_guess", "ssd_saguaro_topf_workspace_bytes", "ssd_saguaro_topf",
           "ssd_saguaro_sample_workspace_bytes", "ssd_saguaro_sample", "ssd_batch_speedup",
           "ssd_backup_crossover",
           "ssd_saguaro_workspace_bytes", "ssd_saguaro_adjust", "ssd_fanout_alloc", "ssd_cache_keys",
           "ssd_cache_lookup", "ssd_read_flags", "ssd_status_string", "ssd_verify_noalloc",
           "ssd_cache_keys_lookup"]

_lib = None
P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64
F32 = ctypes.c_float
F64 = ctypes.c_double
SZ = ctypes.c_size_t


def _declare(L):
    L.ssd_status_string.restype = ctypes.c_char_p
    L.ssd_status_string.argtypes = [ctypes.c_int]
    L.ssd_verify_workspace_bytes.restype = SZ
    L.ssd_verify_workspace_bytes.argtypes = [I32, I32, I32, I32]
    L.ssd_verify_launches.restype = ctypes.c_int
    L.ssd_verify_launches.argtypes = [I32, I32, I32, ctypes.c_int, I32]
    L.ssd_verify_tiles.restype = ctypes.c_int
    L.ssd_verify_tiles.argtypes = [I32, I32, I32, ctypes.c_int]
    L.ssd_verify.restype = ctypes.c_int
    L.ssd_verify.argtypes = [P, I64, P, I64, ctypes.c_int, I32, I32, I32, F32, P, P, P, I32, F32, P,
                             P, I32, P, P, P, P, P, P, SZ, P]
    L.ssd_verify_noalloc.restype = ctypes.c_int
    L.ssd_verify_noalloc.argtypes = [P, I64, P, I64, ctypes.c_int, I32, I32, I32, F32, P, P, P, I32, F32, P,
                                     P, I32, P, P, P, P, P, P, P]
    L.ssd_verify_ex.restype = ctypes.c_int
    L.ssd_verify_ex.argtypes = [P, I64, P, I64, ctypes.c_int, I32, I32, I32, F32, P, P, P, I32, F32, P,
                                P, I32, P, P, P, P, P, P, P, SZ, P]
    L.ssd_stream_read.restype = ctypes.c_int
    L.ssd_stream_read.argtypes = [P, SZ, P, P]
    L.ssd_topf_workspace_bytes.restype = SZ
    L.ssd_topf_workspace_bytes.argtypes = [I32, I32, I32]
    L.ssd_topf_guess.restype = ctypes.c_int
    L.ssd_topf_guess.argtypes = [P, I64, ctypes.c_int, I32, I32, P, P, I32, P, P, SZ, P]
    L.ssd_saguaro_topf_workspace_bytes.restype = SZ
    L.ssd_saguaro_topf_workspace_bytes.argtypes = [I32, I32, I32]
    L.ssd_saguaro_topf.restype = ctypes.c_int
    L.ssd_saguaro_topf.argtypes = [P, I64, ctypes.c_int, I32, I32, F32, P, I32, F32, P, P, P, P, P, SZ, P]
    D = ctypes.c_double
    L.ssd_batch_speedup.restype = ctypes.c_int
    L.ssd_batch_speedup.argtypes = [D, D, D, D, D, I32, P]
    L.ssd_backup_crossover.restype = ctypes.c_int
    L.ssd_backup_crossover.argtypes = [D, D, D, D, D, D, D, P, P]
    L.ssd_saguaro_sample_workspace_bytes.restype = SZ
    L.ssd_saguaro_sample_workspace_bytes.argtypes = [I32, I32, I32]
    L.ssd_saguaro_sample.restype = ctypes.c_int
    L.ssd_saguaro_sample.argtypes = [P, I64, ctypes.c_int, I32, I32, F32, P, I32, F32, P, P, P, P, P, P, P,
                                     P, SZ, P]
    L.ssd_saguaro_workspace_bytes.restype = SZ
    L.ssd_saguaro_workspace_bytes.argtypes = [I32, I32]
    L.ssd_saguaro_adjust.restype = ctypes.c_int
    L.ssd_saguaro_adjust.argtypes = [P, I64, ctypes.c_int, I32, I32, F32, P, I32, F32, P, P, P, P, P,
                                     SZ, P]
    L.ssd_fanout_alloc.restype = ctypes.c_int
    L.ssd_fanout_alloc.argtypes = [I32, F64, F64, I32, P, P]
    L.ssd_cache_keys.restype = ctypes.c_int
    L.ssd_cache_keys.argtypes = [I32, I32, I32, P, P, I32, P, I32, P, P, P]
    L.ssd_cache_keys_lookup.restype = ctypes.c_int
    L.ssd_cache_keys_lookup.argtypes = [I32, I32, I32, P, P, I32, P, I32, P, P, P, P, P, P, P]
    L.ssd_cache_lookup.restype = ctypes.c_int
    L.ssd_cache_lookup.argtypes = [I32, I32, P, P, P, P, P, P, P]
    L.ssd_read_flags.restype = ctypes.c_int
    L.ssd_read_flags.argtypes = [P, P, ctypes.c_int, P]


_lib_path = LIB_PATH


def use_trace_library() -> None:
    """Load libssd_trace.so (ssd_verify with per-workgroup phase timestamps) instead of libssd.so.
    Analysis only; must come before the first call."""
    global _lib_path
    if _lib is not None and _lib_path != TRACE_LIB_PATH:
        raise RuntimeError("the library is already loaded")
    _lib_path = TRACE_LIB_PATH


def lib():
    """The loaded library. Raises if it is missing: there is no CPU or Python fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(_lib_path):
            raise RuntimeError(f"{_lib_path} is not built; run `python -m draft_verification_ssd_amd.build`")
        L = ctypes.CDLL(_lib_path)
        _declare(L)
        if _lib_path == TRACE_LIB_PATH:
            L.ssd_set_trace_buffer.restype = None
            L.ssd_set_trace_buffer.argtypes = [P]
        _lib = L
    return _lib


def check(status: int, what: str) -> None:
    if status != SSD_OK:
        msg = lib().ssd_status_string(status).decode()
        raise RuntimeError(f"{what} failed: status {status} ({msg})")


# ------------------------------------------------------------------------------------------------
# torch helpers (marshalling only)
# ------------------------------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream, device=None) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SSD_F32
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _need(t, dtype, shape, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous with shape {tuple(shape)}, got {tuple(t.shape)}")


def _rows3(t, name, min_rows):
    """[B, rows, V] logits with unit element stride and row stride V; returns (B, rows, V, seq stride)."""
    if t.dim() != 3 or not t.is_cuda:
        raise ValueError(f"{name} must be a 3-d device tensor")
    B, rows, V = t.shape
    if t.stride(2) != 1 or (rows > 1 and t.stride(1) != V) or rows < min_rows:
        raise ValueError(f"{name}: rows must be contiguous V-vectors, at least {min_rows} per sequence")
    return B, rows, V, (t.stride(0) if B > 1 else rows * V)


class Workspace:
    """Zero-initialised device scratch, 256-byte aligned (torch's allocator guarantees it)."""

    def __init__(self, nbytes: int, device=None):
        torch = _torch()
        self.nbytes = int(max(nbytes, 256))
        self.buf = torch.zeros(self.nbytes, dtype=torch.uint8, device=device or "cuda")
        if self.buf.data_ptr() % 256:
            raise RuntimeError("workspace is not 256-byte aligned")

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr()


def ssd_verify_workspace_bytes(B: int, K: int, V: int, topf_F_max: int = 0) -> int:
    return int(lib().ssd_verify_workspace_bytes(B, K, V, topf_F_max))


def ssd_verify_launches(B: int, K: int, V: int, dtype: int, topf_F_max: int = 0) -> int:
    """Kernel launches ssd_verify issues for this shape on the current device: 2 (the streaming
    form) when the batch has more tiles than the device runs at once, else 1 (-1 if rejected)."""
    return int(lib().ssd_verify_launches(B, K, V, dtype, topf_F_max))


def ssd_verify_tiles(B: int, K: int, V: int, dtype: int) -> int:
    """Tiles per logit row (workgroups per sequence) ssd_verify takes for this shape (-1 if rejected)."""
    return int(lib().ssd_verify_tiles(B, K, V, dtype))


def ssd_stream_read(data, sink, stream=None) -> None:
    """Measurement helper: read every byte of a device tensor once (sink: device int32 [8192])."""
    nbytes = data.numel() * data.element_size()
    check(lib().ssd_stream_read(data.data_ptr(), nbytes, sink.data_ptr(), _stream(stream, data.device)),
          "ssd_stream_read")


def ssd_topf_workspace_bytes(R: int, V: int, F_max: int) -> int:
    return int(lib().ssd_topf_workspace_bytes(R, V, F_max))


def ssd_saguaro_topf_workspace_bytes(R: int, V: int, F_max: int) -> int:
    return int(lib().ssd_saguaro_topf_workspace_bytes(R, V, F_max))


def ssd_saguaro_sample_workspace_bytes(R: int, V: int, F_max: int) -> int:
    return int(lib().ssd_saguaro_sample_workspace_bytes(R, V, F_max))


def ssd_saguaro_workspace_bytes(R: int, V: int) -> int:
    return int(lib().ssd_saguaro_workspace_bytes(R, V))


def ssd_read_flags(workspace: Workspace, clear: bool = True, stream=None) -> int:
    out = ctypes.c_uint32(0)
    check(lib().ssd_read_flags(workspace.ptr, ctypes.addressof(out), int(clear), _stream(stream)),
          "ssd_read_flags")
    return int(out.value)


# ------------------------------------------------------------------------------------------------
class VerifyCall:
    """A fully marshalled ssd_verify call: building it validates shapes once; calling it issues one
    foreign call with the stored arguments (the launch path used for timing)."""

    def __init__(self, draft, target, draft_tokens, uniforms, temperature: float, *,
                 sag_set=None, sag_C=1.0, topf_F: Optional[Sequence[int]] = None,
                 topf_F_max: int = 0, topf_out=None, accepted_len=None, bonus_token=None,
                 accept_prob=None, residual_mass=None, workspace: Optional[Workspace] = None,
                 stream=None, wait_polls: Optional[int] = None, topf_last_F: int = 0, topf_last_out=None,
                 noalloc_flags=None, launch_mode: int = 0):
        torch = _torch()
        B, Kd, V, dstride = _rows3(draft, "draft", 1)
        Bt, Kt, Vt, tstride = _rows3(target, "target", 2)
        K = Kt - 1
        if Bt != B or Vt != V or Kd < K or draft.dtype != target.dtype:
            raise ValueError("draft [B, >=K, V] and target [B, K+1, V] must agree")
        dev = draft.device
        _need(draft_tokens, torch.int32, (B, K), "draft_tokens")
        _need(uniforms, torch.float32, (B, K + 1), "uniforms")
        sag_F = 0
        if sag_set is not None:
            if sag_set.dim() != 3 or tuple(sag_set.shape[:2]) != (B, K):
                raise ValueError("sag_set must be [B, K, F]")
            sag_F = int(sag_set.shape[2])
            _need(sag_set, torch.int32, (B, K, sag_F), "sag_set")
        if topf_F_max > 0:
            if topf_out is None:
                topf_out = torch.empty((B, K, topf_F_max), dtype=torch.int32, device=dev)
            _need(topf_out, torch.int32, (B, K, topf_F_max), "topf_out")
        self.sag_C_arr = None  # per-position C, host [K]
        if sag_set is not None and not isinstance(sag_C, (int, float)):
            cs = [float(c) for c in sag_C]
            if len(cs) != K:
                raise ValueError("sag_C needs one value or one per draft position")
            self.sag_C_arr = (ctypes.c_float * K)(*cs)
            sag_C = cs[0]
        elif not isinstance(sag_C, (int, float)):
            sag_C = float(list(sag_C)[0])
        self.topf_F_arr = None
        if topf_F is not None:
            if len(topf_F) != K:
                raise ValueError("topf_F needs one entry per draft position")
            self.topf_F_arr = (ctypes.c_int32 * K)(*[int(f) for f in topf_F])
        if accepted_len is None:
            accepted_len = torch.empty(B, dtype=torch.int32, device=dev)
        if bonus_token is None:
            bonus_token = torch.empty(B, dtype=torch.int32, device=dev)
        _need(accepted_len, torch.int32, (B,), "accepted_len")
        _need(bonus_token, torch.int32, (B,), "bonus_token")
        if accept_prob is not None:
            _need(accept_prob, torch.float32, (B, K), "accept_prob")
        if residual_mass is not None:
            _need(residual_mass, torch.float32, (B,), "residual_mass")
        if topf_last_F > 0:
            if topf_last_out is None:
                topf_last_out = torch.empty((B, topf_last_F), dtype=torch.int32, device=dev)
            _need(topf_last_out, torch.int32, (B, topf_last_F), "topf_last_out")
        self.opts = None
        if wait_polls is not None or topf_last_F > 0 or launch_mode != 0:
            self.opts = VerifyOpts(-1 if wait_polls is None else int(wait_polls), int(topf_last_F),
                                   _ptr(topf_last_out) if topf_last_F > 0 else None, int(launch_mode))
        if noalloc_flags is not None:  # ssd_verify_noalloc: the library's static workspace
            if self.opts is not None or workspace is not None:
                raise ValueError("noalloc_flags excludes workspace, wait_polls, topf_last_F and launch_mode")
            _need(noalloc_flags, torch.int32, (1,), "noalloc_flags")
        elif workspace is None:
            workspace = Workspace(ssd_verify_workspace_bytes(B, K, V, max(topf_F_max, topf_last_F)), dev)
        self.B, self.K, self.V = B, K, V
        self.workspace = workspace
        self.outputs = dict(accepted_len=accepted_len, bonus_token=bonus_token, accept_prob=accept_prob,
                            residual_mass=residual_mass, topf=topf_out, topf_last=topf_last_out)
        self._keep = (draft, target, draft_tokens, uniforms, sag_set)
        self.args = (
            draft.data_ptr(), dstride, target.data_ptr(), tstride, _dtype_code(draft), B, K, V,
            float(temperature), draft_tokens.data_ptr(), uniforms.data_ptr(), _ptr(sag_set), sag_F,
            float(sag_C), None if self.sag_C_arr is None else ctypes.addressof(self.sag_C_arr),
            None if self.topf_F_arr is None else ctypes.addressof(self.topf_F_arr), int(topf_F_max),
            _ptr(topf_out), accepted_len.data_ptr(), bonus_token.data_ptr(), _ptr(accept_prob),
            _ptr(residual_mass), None if workspace is None else workspace.ptr,
            0 if workspace is None else workspace.nbytes, _stream(stream, dev))
        if noalloc_flags is not None:
            self.args = self.args[:22] + (noalloc_flags.data_ptr(), self.args[24])
            self._keep = self._keep + (noalloc_flags,)
            self._fn = lib().ssd_verify_noalloc
        elif self.opts is not None:
            self.args = self.args[:22] + (ctypes.addressof(self.opts),) + self.args[22:]
            self._fn = lib().ssd_verify_ex
        else:
            self._fn = lib().ssd_verify

    def __call__(self):
        check(self._fn(*self.args), "ssd_verify")
        return self.outputs

    def flags(self, clear: bool = True) -> int:
        """Device-error flags of this call's workspace (synchronises the stream)."""
        if self.workspace is None:
            raise ValueError("an allocation-free call reports its flags in its noalloc_flags word")
        return ssd_read_flags(self.workspace, clear)

    def checked(self):
        """Run, synchronise and raise if the device recorded an error (SSD_FLAG_*)."""
        out = self()
        f = self.flags()
        if f:
            raise RuntimeError(f"ssd_verify: device flags {f:#x}")
        return out


def ssd_verify(draft, target, draft_tokens, uniforms, temperature: float, **kw):
    """Verify one round for B sequences; returns the output tensors (see include/ssd.h)."""
    return VerifyCall(draft, target, draft_tokens, uniforms, temperature, **kw)()


def ssd_topf_guess(logits, F_max: int, *, exclude=None, F_per_row=None, out=None,
                   workspace: Optional[Workspace] = None, stream=None):
    """Top-F guesses of every row of a [R, V] (or [..., V] with row stride) logits view."""
    torch = _torch()
    if logits.dim() != 2 or logits.stride(1) != 1 or not logits.is_cuda:
        raise ValueError("logits must be a [R, V] device view with unit element stride")
    R, V = logits.shape
    dev = logits.device
    if exclude is not None:
        _need(exclude, torch.int32, (R,), "exclude")
    if F_per_row is not None:
        _need(F_per_row, torch.int32, (R,), "F_per_row")
    if out is None:
        out = torch.empty((R, F_max), dtype=torch.int32, device=dev)
    _need(out, torch.int32, (R, F_max), "out")
    if workspace is None:
        workspace = Workspace(ssd_topf_workspace_bytes(R, V, F_max), dev)
    stride = logits.stride(0) if R > 1 else V
    check(lib().ssd_topf_guess(logits.data_ptr(), stride, _dtype_code(logits), R, V, _ptr(exclude),
                               _ptr(F_per_row), F_max, out.data_ptr(), workspace.ptr,
                               workspace.nbytes, _stream(stream, dev)), "ssd_topf_guess")
    return out


def ssd_saguaro_adjust(logits, temperature: float, set_, C: float, *, C_per_row=None,
                       materialise: bool = False, out_probs=None, out_set_mass=None, out_norm=None,
                       workspace: Optional[Workspace] = None, stream=None):
    """Saguaro down-weighting of every row of a [R, V] logits view; returns (q' or None, sigma, N).
    C_per_row: optional device fp32 [R] factor per row."""
    torch = _torch()
    if logits.dim() != 2 or logits.stride(1) != 1 or not logits.is_cuda:
        raise ValueError("logits must be a [R, V] device view with unit element stride")
    R, V = logits.shape
    dev = logits.device
    F = 0
    if set_ is not None:
        F = int(set_.shape[1])
        _need(set_, torch.int32, (R, F), "set")
    if materialise and out_probs is None:
        out_probs = torch.empty((R, V), dtype=torch.float32, device=dev)
    if out_probs is not None:
        _need(out_probs, torch.float32, (R, V), "out_probs")
    if out_set_mass is None:
        out_set_mass = torch.empty(R, dtype=torch.float32, device=dev)
    if out_norm is None:
        out_norm = torch.empty(R, dtype=torch.float32, device=dev)
    _need(out_set_mass, torch.float32, (R,), "out_set_mass")
    _need(out_norm, torch.float32, (R,), "out_norm")
    if workspace is None:
        workspace = Workspace(ssd_saguaro_workspace_bytes(R, V), dev)
    stride = logits.stride(0) if R > 1 else V
    if C_per_row is not None:
        _need(C_per_row, torch.float32, (R,), "C_per_row")
    check(lib().ssd_saguaro_adjust(logits.data_ptr(), stride, _dtype_code(logits), R, V,
                                   float(temperature), _ptr(set_), F, float(C), _ptr(C_per_row), _ptr(out_probs),
                                   out_set_mass.data_ptr(), out_norm.data_ptr(), workspace.ptr,
                                   workspace.nbytes, _stream(stream, dev)), "ssd_saguaro_adjust")
    return out_probs, out_set_mass, out_norm


def ssd_saguaro_topf(logits, temperature: float, F_max: int, C: float, *, F_per_row=None, C_per_row=None,
                     out_set=None, out_set_mass=None, out_norm=None, workspace: Optional[Workspace] = None,
                     stream=None):
    """Each row's top-F set with its Saguaro mass and normaliser in one pass; returns (set, sigma, N).
    C_per_row: optional device fp32 [R] factor per row."""
    torch = _torch()
    if logits.dim() != 2 or logits.stride(1) != 1 or not logits.is_cuda:
        raise ValueError("logits must be a [R, V] device view with unit element stride")
    R, V = logits.shape
    dev = logits.device
    if F_per_row is not None:
        _need(F_per_row, torch.int32, (R,), "F_per_row")
    if out_set is None:
        out_set = torch.empty((R, F_max), dtype=torch.int32, device=dev)
    if out_set_mass is None:
        out_set_mass = torch.empty(R, dtype=torch.float32, device=dev)
    if out_norm is None:
        out_norm = torch.empty(R, dtype=torch.float32, device=dev)
    _need(out_set, torch.int32, (R, F_max), "out_set")
    _need(out_set_mass, torch.float32, (R,), "out_set_mass")
    _need(out_norm, torch.float32, (R,), "out_norm")
    if workspace is None:
        workspace = Workspace(ssd_saguaro_topf_workspace_bytes(R, V, F_max), dev)
    stride = logits.stride(0) if R > 1 else V
    if C_per_row is not None:
        _need(C_per_row, torch.float32, (R,), "C_per_row")
    check(lib().ssd_saguaro_topf(logits.data_ptr(), stride, _dtype_code(logits), R, V, float(temperature),
                                 _ptr(F_per_row), int(F_max), float(C), _ptr(C_per_row), out_set.data_ptr(),
                                 out_set_mass.data_ptr(), out_norm.data_ptr(), workspace.ptr, workspace.nbytes,
                                 _stream(stream, dev)), "ssd_saguaro_topf")
    return out_set, out_set_mass, out_norm


def ssd_saguaro_sample(logits, temperature: float, F_max: int, C: float, u, *, F_per_row=None,
                       C_per_row=None, out_token=None, out_prob=None, out_set=None, out_set_mass=None,
                       out_norm=None, workspace: Optional[Workspace] = None, stream=None):
    """The draft's sampling step with Saguaro: each row's top-F set, its mass and normaliser, and a
    token drawn from the down-weighted distribution with the row's uniform u (device fp32 [R]) in
    one pass; returns (token, q' of it, set, sigma, N)."""
    torch = _torch()
    if logits.dim() != 2 or logits.stride(1) != 1 or not logits.is_cuda:
        raise ValueError("logits must be a [R, V] device view with unit element stride")
    R, V = logits.shape
    dev = logits.device
    _need(u, torch.float32, (R,), "u")
    if F_per_row is not None:
        _need(F_per_row, torch.int32, (R,), "F_per_row")
    if C_per_row is not None:
        _need(C_per_row, torch.float32, (R,), "C_per_row")
    if out_token is None:
        out_token = torch.empty(R, dtype=torch.int32, device=dev)
    if out_prob is None:
        out_prob = torch.empty(R, dtype=torch.float32, device=dev)
    if out_set is None:
        out_set = torch.empty((R, F_max), dtype=torch.int32, device=dev)
    if out_set_mass is None:
        out_set_mass = torch.empty(R, dtype=torch.float32, device=dev)
    if out_norm is None:
        out_norm = torch.empty(R, dtype=torch.float32, device=dev)
    _need(out_token, torch.int32, (R,), "out_token")
    _need(out_prob, torch.float32, (R,), "out_prob")
    _need(out_set, torch.int32, (R, F_max), "out_set")
    _need(out_set_mass, torch.float32, (R,), "out_set_mass")
    _need(out_norm, torch.float32, (R,), "out_norm")
    if workspace is None:
        workspace = Workspace(ssd_saguaro_sample_workspace_bytes(R, V, F_max), dev)
    stride = logits.stride(0) if R > 1 else V
    check(lib().ssd_saguaro_sample(logits.data_ptr(), stride, _dtype_code(logits), R, V, float(temperature),
                                   _ptr(F_per_row), int(F_max), float(C), _ptr(C_per_row), u.data_ptr(),
                                   out_token.data_ptr(), out_prob.data_ptr(), _ptr(out_set if F_max > 0 else None),
                                   out_set_mass.data_ptr(), out_norm.data_ptr(), workspace.ptr, workspace.nbytes,
                                   _stream(stream, dev)), "ssd_saguaro_sample")
    return out_token, out_prob, out_set, out_set_mass, out_norm


def ssd_batch_speedup(h: float, E_hit: float, E_miss: float, T_p: float, T_b: float, b: int) -> float:
    """Host-only expected speedup of a batch of b sequences under cache misses."""
    out = ctypes.c_double()
    check(lib().ssd_batch_speedup(h, E_hit, E_miss, T_p, T_b, int(b), ctypes.byref(out)), "ssd_batch_speedup")
    return out.value


def ssd_backup_crossover(h: float, E_hit: float, E_miss_neural: float, T_neural: float, E_miss_fast: float,
                         T_fast: float, T_p: float):
    """Host-only batch size where the fast and neural backups tie; returns (b_star, fast_wins_large)."""
    b = ctypes.c_double()
    f = ctypes.c_int32()
    check(lib().ssd_backup_crossover(h, E_hit, E_miss_neural, T_neural, E_miss_fast, T_fast, T_p, ctypes.byref(b),
                                     ctypes.byref(f)), "ssd_backup_crossover")
    return b.value, bool(f.value)


def ssd_fanout_alloc(K: int, a: float, r: float, budget: int):
    """Host-only geometric fan-out; returns (list of K+1 ints, list of K+1 floats)."""
    F = (ctypes.c_int32 * (K + 1))()
    Fc = (ctypes.c_double * (K + 1))()
    check(lib().ssd_fanout_alloc(K, a, r, budget, ctypes.addressof(F), ctypes.addressof(Fc)),
          "ssd_fanout_alloc")
    return list(F), list(Fc)


def ssd_cache_keys(guesses, fanout: Sequence[int], *, guesses_last=None, cache_k=None, cache_tok=None,
                   stream=None):
    """guesses [B, K+1, G_max] int32 device, or [B, K, G_max] (ssd_verify's top-F output) with
    guesses_last [B, G_last] (position K's, ssd_topf_guess's output) -> (cache_k, cache_tok) [B, budget]."""
    torch = _torch()
    B, Kg, G = guesses.shape
    _need(guesses, torch.int32, (B, Kg, G), "guesses")
    K = Kg if guesses_last is not None else Kg - 1
    K1 = K + 1
    G_last = 0
    if guesses_last is not None:
        G_last = guesses_last.shape[1]
        _need(guesses_last, torch.int32, (B, G_last), "guesses_last")
    budget = int(sum(int(f) for f in fanout))
    dev = guesses.device
    if cache_k is None:
        cache_k = torch.empty((B, budget), dtype=torch.int32, device=dev)
    if cache_tok is None:
        cache_tok = torch.empty((B, budget), dtype=torch.int32, device=dev)
    F = (ctypes.c_int32 * K1)(*[int(f) for f in fanout])
    check(lib().ssd_cache_keys(B, K, G, guesses.data_ptr(), _ptr(guesses_last), G_last, ctypes.addressof(F), budget,
                               cache_k.data_ptr(), cache_tok.data_ptr(), _stream(stream, dev)),
          "ssd_cache_keys")
    return cache_k, cache_tok


def ssd_cache_lookup(cache_k, cache_tok, accepted_len, bonus_token, *, out_slot=None,
                     out_miss_count=None, stream=None):
    """Returns (slot [B] int32, miss count [1] int32), both on the device."""
    torch = _torch()
    B, budget = cache_k.shape
    dev = cache_k.device
    _need(cache_k, torch.int32, (B, budget), "cache_k")
    _need(cache_tok, torch.int32, (B, budget), "cache_tok")
    _need(accepted_len, torch.int32, (B,), "accepted_len")
    _need(bonus_token, torch.int32, (B,), "bonus_token")
    if out_slot is None:
        out_slot = torch.empty(B, dtype=torch.int32, device=dev)
    if out_miss_count is None:
        out_miss_count = torch.empty(1, dtype=torch.int32, device=dev)
    check(lib().ssd_cache_lookup(B, budget, cache_k.data_ptr(), cache_tok.data_ptr(),
                                 accepted_len.data_ptr(), bonus_token.data_ptr(), out_slot.data_ptr(),
                                 out_miss_count.data_ptr(), _stream(stream, dev)), "ssd_cache_lookup")
    return out_slot, out_miss_count


def ssd_cache_keys_lookup(guesses, fanout: Sequence[int], accepted_len, bonus_token, *, guesses_last=None,
                          cache_k=None, cache_tok=None, out_slot=None, out_miss_count=None, stream=None):
    """ssd_cache_keys and ssd_cache_lookup in one launch; returns (cache_k, cache_tok, slot, miss count)."""
    torch = _torch()
    B, Kg, G = guesses.shape
    _need(guesses, torch.int32, (B, Kg, G), "guesses")
    K = Kg if guesses_last is not None else Kg - 1
    G_last = 0
    if guesses_last is not None:
        G_last = guesses_last.shape[1]
        _need(guesses_last, torch.int32, (B, G_last), "guesses_last")
    _need(accepted_len, torch.int32, (B,), "accepted_len")
    _need(bonus_token, torch.int32, (B,), "bonus_token")
    budget = int(sum(int(f) for f in fanout))
    dev = guesses.device
    if cache_k is None:
        cache_k = torch.empty((B, budget), dtype=torch.int32, device=dev)
    if cache_tok is None:
        cache_tok = torch.empty((B, budget), dtype=torch.int32, device=dev)
    if out_slot is None:
        out_slot = torch.empty(B, dtype=torch.int32, device=dev)
    if out_miss_count is None:
        out_miss_count = torch.empty(1, dtype=torch.int32, device=dev)
    F = (ctypes.c_int32 * (K + 1))(*[int(f) for f in fanout])
    check(lib().ssd_cache_keys_lookup(B, K, G, guesses.data_ptr(), _ptr(guesses_last), G_last, ctypes.addressof(F),
                                      budget, accepted_len.data_ptr(), bonus_token.data_ptr(), cache_k.data_ptr(),
                                      cache_tok.data_ptr(), out_slot.data_ptr(), out_miss_count.data_ptr(),
                                      _stream(stream, dev)), "ssd_cache_keys_lookup")
    return cache_k, cache_tok, out_slot, out_miss_count
