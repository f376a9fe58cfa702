"""Thin ctypes binding of libxattn (include/xattn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the stream;
host scalars (request, candidate and memory-row counts) come from tensor
shapes, so no call synchronises with the device.  The library is loaded on
first use and a missing build raises ``RuntimeError`` - there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.environ.get("XATTN_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libxattn.so")
_lib = None

XATTN_OK, XATTN_EINVAL, XATTN_EUNSUPPORTED, XATTN_EHIP, XATTN_EWORKSPACE = 0, -1, -2, -3, -4
XATTN_EDEVICE_VALIDATION = -5
XATTN_BF16, XATTN_FP32 = 0, 1
XATTN_KV_SHARED, XATTN_KV_SEPARATE = 0, 1

EXPORTED = ("xattn_create", "xattn_destroy", "xattn_workspace_size", "xattn_forward",
            "xattn_attend", "xattn_attend_q", "xattn_plan", "xattn_max_tiles",
            "xattn_forward_launches", "xattn_project", "xattn_output", "xattn_device_error",
            "xattn_last_error", "xattn_forward_prefix", "xattn_attend_q_prefix",
            "xattn_backward_workspace_size", "xattn_backward", "xattn_codec_encode",
            "xattn_codec_fold_query_weights", "xattn_forward_codec", "xattn_forward_path",
            "xattn_codec_workspace_size", "xattn_forward_train", "xattn_backward_saved",
            "xattn_forward_noalloc", "xattn_codec_fit")

# include/xattn.h: bytes of the library-owned scratch of xattn_forward_noalloc
NOALLOC_SCRATCH_BYTES = 32 << 20

# xattn_path values (include/xattn.h)
PATH_SINGLE, PATH_GEMM, PATH_FP32, PATH_SHORT = 1, 2, 3, 4


class CodebookStruct(ctypes.Structure):
    _fields_ = [("budget_bits", ctypes.c_int32), ("bits", ctypes.c_void_p),
                ("center", ctypes.c_void_p), ("half_range", ctypes.c_void_p),
                ("rotation", ctypes.c_void_p)]


class Codebook:
    """Device-resident codebook of a coded memory (see include/xattn.h):
    bits uint8 [heads, d_h], center/half_range/rotation fp32.  The tensors are
    kept alive by this object."""

    def __init__(self, bits, center, half_range, rotation, budget_bits: int, device="cuda"):
        t = lambda a, dt: torch.as_tensor(a).to(device=device, dtype=dt).contiguous()
        self.bits = t(bits, torch.uint8)
        self.center = t(center, torch.float32)
        self.half_range = t(half_range, torch.float32)
        self.rotation = t(rotation, torch.float32)
        self.budget_bits = int(budget_bits)
        self.heads, self.d_h = self.bits.shape

    @property
    def words(self) -> int:
        return self.budget_bits // 32

    def struct(self) -> CodebookStruct:
        return CodebookStruct(self.budget_bits, self.bits.data_ptr(), self.center.data_ptr(),
                              self.half_range.data_ptr(), self.rotation.data_ptr())


def codec_fit(X, heads: int, budget_bits: int) -> dict:
    """Codebook fitted by the library on the host (xattn_codec_fit) from a
    calibration sample X [n, d] (array-like, read as fp32): dict of bits
    uint8 [heads, d_h], center, half and rot fp32, budget (what Codebook
    takes)."""
    import numpy as np
    Xh = np.ascontiguousarray(np.asarray(X, dtype=np.float32))
    n, d = Xh.shape
    dh = d // heads
    bits = np.zeros((heads, dh), dtype=np.uint8)
    center = np.zeros((heads, dh), dtype=np.float32)
    half = np.zeros((heads, dh), dtype=np.float32)
    rot = np.zeros((heads, dh, dh), dtype=np.float32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    st = lib().xattn_codec_fit(d, heads, p(Xh), n, int(budget_bits), p(bits), p(center), p(half),
                               p(rot))
    if st != XATTN_OK:
        raise XAttnError(st, "xattn_codec_fit rejected its arguments")
    return {"bits": bits, "center": center, "half": half, "rot": rot, "budget": int(budget_bits)}


class Config(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_slots", ctypes.c_int32),
                ("dtype", ctypes.c_int), ("kv_mode", ctypes.c_int), ("device", ctypes.c_int32)]


class XAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("xattn status %d: %s" % (status, msg))
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load libxattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libxattn.so is not built (%s); run "
                               "`python -m shared_history_candidate_amd.build`" % _LIB_PATH)
        L = ctypes.CDLL(_LIB_PATH)
        P, I32, SZ, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_int64
        L.xattn_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(P)]
        L.xattn_create.restype = ctypes.c_int
        L.xattn_destroy.argtypes = [P]
        L.xattn_destroy.restype = None
        L.xattn_workspace_size.argtypes = [P, I32, I32, I32]
        L.xattn_workspace_size.restype = SZ
        L.xattn_codec_workspace_size.argtypes = [P, I32, I32, I32, I32]
        L.xattn_codec_workspace_size.restype = SZ
        L.xattn_max_tiles.argtypes = [P, I32, I32, I32]
        L.xattn_max_tiles.restype = I64
        L.xattn_forward_launches.argtypes = [P, I32, I32, I32, I32]
        L.xattn_forward_launches.restype = I32
        L.xattn_forward_path.argtypes = [P, I32, I32, I32, I32]
        L.xattn_forward_path.restype = I32
        L.xattn_forward.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, P, P, SZ, P]
        L.xattn_forward.restype = ctypes.c_int
        L.xattn_forward_noalloc.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, P, P]
        L.xattn_forward_noalloc.restype = ctypes.c_int
        L.xattn_forward_prefix.argtypes = [P, P, P, P, P, P, P, P, I32, I32, I32, I32, P, P, SZ,
                                           P]
        L.xattn_forward_prefix.restype = ctypes.c_int
        L.xattn_attend.argtypes = L.xattn_forward.argtypes
        L.xattn_attend.restype = ctypes.c_int
        L.xattn_attend_q.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, P, P, SZ, P]
        L.xattn_attend_q.restype = ctypes.c_int
        L.xattn_attend_q_prefix.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, P, P, SZ, P]
        L.xattn_attend_q_prefix.restype = ctypes.c_int
        L.xattn_backward_workspace_size.argtypes = [P, I32, I32, I32, I32]
        L.xattn_backward_workspace_size.restype = SZ
        L.xattn_backward.argtypes = [P, P, P, P, P, P, P, P, P, I32, I32, I32, I32, P, P, P, P,
                                     P, SZ, P]
        L.xattn_backward.restype = ctypes.c_int
        L.xattn_forward_train.argtypes = [P, P, P, P, P, P, P, P, I32, I32, I32, I32, P, P, P, SZ,
                                          P]
        L.xattn_forward_train.restype = ctypes.c_int
        L.xattn_backward_saved.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I32, I32, I32, I32, P,
                                           P, P, P, P, SZ, P]
        L.xattn_backward_saved.restype = ctypes.c_int
        CB = ctypes.POINTER(CodebookStruct)
        L.xattn_codec_fit.argtypes = [I32, I32, P, I64, I32, P, P, P, P]
        L.xattn_codec_fit.restype = ctypes.c_int
        L.xattn_codec_encode.argtypes = [P, CB, I32, P, I32, P, P, P]
        L.xattn_codec_encode.restype = ctypes.c_int
        L.xattn_codec_fold_query_weights.argtypes = [P, CB, I32, P, P, P]
        L.xattn_codec_fold_query_weights.restype = ctypes.c_int
        L.xattn_forward_codec.argtypes = [P, CB, CB, P, P, P, P, P, P, P, P, I32, I32, I32, I32, P,
                                          P, SZ, P]
        L.xattn_forward_codec.restype = ctypes.c_int
        L.xattn_plan.argtypes = [P, P, P, I32, I32, I32, I32, P, P, P, P,
                                 ctypes.POINTER(I32), P, SZ, P]
        L.xattn_plan.restype = ctypes.c_int
        L.xattn_project.argtypes = [P, P, P, I32, P, P]
        L.xattn_output.argtypes = [P, P, P, P, P, I32, P, P, ctypes.c_size_t, P]
        L.xattn_output.restype = ctypes.c_int
        L.xattn_project.restype = ctypes.c_int
        L.xattn_device_error.argtypes = [P, P, ctypes.POINTER(I32), P]
        L.xattn_device_error.restype = ctypes.c_int
        L.xattn_last_error.argtypes = []
        L.xattn_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != XATTN_OK:
        raise XAttnError(status, lib().xattn_last_error().decode())


class BoundCall:
    """One C-ABI call with its arguments marshalled once (tensors by data
    pointer, scalars as ctypes values).  Calling it makes the same call again
    and raises on a non-OK status.  For tight timing loops, where the per-call
    argument checks of the methods below would leave host gaps between short
    kernels; the caller keeps the tensors alive."""

    def __init__(self, fn, args):
        self._fn = fn
        self._args = tuple(args)

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != XATTN_OK:
            _check(st)


def _call(fn, args, bind: bool):
    """Call fn(*args), or return it as a BoundCall when bind is set."""
    if bind:
        return BoundCall(fn, args)
    _check(fn(*args))
    return None


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


_DTYPES = {"bf16": (XATTN_BF16, torch.bfloat16), "fp32": (XATTN_FP32, torch.float32)}
_MODES = {"shared": XATTN_KV_SHARED, "separate": XATTN_KV_SEPARATE}


class XAttn:
    """One library context: fixed d_model, q (slots), dtype and K/V mode."""

    def __init__(self, d_model: int, n_slots: int, dtype: str = "bf16", kv_mode: str = "shared",
                 device: int = 0):
        if dtype not in _DTYPES or kv_mode not in _MODES:
            raise ValueError("dtype must be bf16|fp32 and kv_mode shared|separate")
        self.d_model, self.q, self.dtype_name, self.kv_mode = d_model, n_slots, dtype, kv_mode
        self.torch_dtype = _DTYPES[dtype][1]
        self.device = device
        cfg = Config(d_model, n_slots, _DTYPES[dtype][0], _MODES[kv_mode], device)
        h = ctypes.c_void_p()
        _check(lib().xattn_create(ctypes.byref(cfg), ctypes.byref(h)))
        self._h = h

    def close(self) -> None:
        if getattr(self, "_h", None):
            lib().xattn_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- sizes ---------------------------------------------------------------
    def workspace_size(self, num_requests: int, total_cand: int, heads: int) -> int:
        return int(lib().xattn_workspace_size(self._h, num_requests, total_cand, heads))

    def codec_workspace_size(self, num_requests: int, total_cand: int, total_kv: int,
                             heads: int) -> int:
        """Workspace bytes with room for the decoded memory (xattn_forward_codec
        decodes the memory once per call)."""
        return int(lib().xattn_codec_workspace_size(self._h, num_requests, total_cand, total_kv,
                                                    heads))

    def max_tiles(self, num_requests: int, total_cand: int, heads: int) -> int:
        return int(lib().xattn_max_tiles(self._h, num_requests, total_cand, heads))

    def forward_launches(self, num_requests: int, total_cand: int, total_kv: int,
                         heads: int) -> int:
        """Kernel launches xattn_forward enqueues for this batch shape."""
        return int(lib().xattn_forward_launches(self._h, num_requests, total_cand, total_kv,
                                                heads))

    def forward_path(self, num_requests: int, total_cand: int, total_kv: int, heads: int) -> int:
        """Which kernels xattn_forward runs for this batch shape (PATH_*)."""
        return int(lib().xattn_forward_path(self._h, num_requests, total_cand, total_kv, heads))

    def alloc_workspace(self, num_requests: int, total_cand: int, heads: int) -> torch.Tensor:
        n = self.workspace_size(num_requests, total_cand, heads)
        return torch.empty(max(n, 256), dtype=torch.uint8, device="cuda:%d" % self.device)

    def _check_tensor(self, name, t, dtype, shape=None):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError("%s must be a CUDA tensor" % name)
        if t.dtype != dtype:
            raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError("%s must have shape %s, got %s" % (name, shape, tuple(t.shape)))

    # -- entry points ----------------------------------------------------------
    def forward(self, Z, W_Q, K, V, cu_seqlens_kv, cu_cand, heads: int, O=None,
                workspace=None, stream=None, plan: bool = True,
                cand_kv_len=None, bind: bool = False) -> torch.Tensor:
        """O = cross-attention of Z's query tokens against their requests' memory
        (see include/xattn.h).  Z [total_cand, q, d], W_Q [q, d, d] output-major,
        K [total_kv, d] (= H), V [total_kv, d] or None, cu_* int32 [R+1].
        cand_kv_len (int32 [total_cand], optional): candidate c sees only the
        first cand_kv_len[c] memory rows of its request (xattn_forward_prefix).
        With bind=True nothing runs: the checked call comes back as a
        BoundCall (O and workspace must then be given)."""
        d, q, dt = self.d_model, self.q, self.torch_dtype
        total_cand, total_kv = Z.shape[0], K.shape[0]
        R = cu_seqlens_kv.numel() - 1
        self._check_tensor("Z", Z, dt, (total_cand, q, d))
        self._check_tensor("W_Q", W_Q, dt, (q, d, d))
        self._check_tensor("K", K, dt, (total_kv, d))
        if V is not None:
            self._check_tensor("V", V, dt, (total_kv, d))
        self._check_tensor("cu_seqlens_kv", cu_seqlens_kv, torch.int32, (R + 1,))
        self._check_tensor("cu_cand", cu_cand, torch.int32, (R + 1,))
        if bind and (O is None or workspace is None):
            raise ValueError("a bound call needs O and the workspace")
        if O is None:
            O = torch.empty((total_cand, q, d), dtype=dt, device=Z.device)
        self._check_tensor("O", O, dt, (total_cand, q, d))
        if workspace is None:
            if not plan:
                raise ValueError("attend() needs the workspace that holds the batch's plan")
            workspace = self.alloc_workspace(R, total_cand, heads)
        if cand_kv_len is not None:
            if not plan:
                raise ValueError("a per-candidate prefix is only available with planning")
            self._check_tensor("cand_kv_len", cand_kv_len, torch.int32, (total_cand,))
            b = _call(lib().xattn_forward_prefix,
                      (self._h, _ptr(Z), _ptr(W_Q), _ptr(K), _ptr(V), _ptr(cu_seqlens_kv),
                       _ptr(cu_cand), _ptr(cand_kv_len), R, total_cand, total_kv, heads,
                       _ptr(O), _ptr(workspace), workspace.numel(), _stream(Z.device, stream)),
                      bind)
            return b if bind else O
        fn = lib().xattn_forward if plan else lib().xattn_attend
        b = _call(fn, (self._h, _ptr(Z), _ptr(W_Q), _ptr(K), _ptr(V), _ptr(cu_seqlens_kv),
                       _ptr(cu_cand), R, total_cand, total_kv, heads, _ptr(O), _ptr(workspace),
                       workspace.numel(), _stream(Z.device, stream)), bind)
        return b if bind else O

    def forward_noalloc(self, Z, W_Q, K, V, cu_seqlens_kv, cu_cand, heads: int, O=None,
                        stream=None) -> torch.Tensor:
        """forward() without a workspace (xattn_forward_noalloc): the library's
        own device scratch stands in for it, so the call allocates nothing but
        O (when O is not given).  Calls that may overlap on one GPU race on
        that scratch."""
        d, q, dt = self.d_model, self.q, self.torch_dtype
        total_cand, total_kv = Z.shape[0], K.shape[0]
        R = cu_seqlens_kv.numel() - 1
        self._check_tensor("Z", Z, dt, (total_cand, q, d))
        self._check_tensor("W_Q", W_Q, dt, (q, d, d))
        self._check_tensor("K", K, dt, (total_kv, d))
        if V is not None:
            self._check_tensor("V", V, dt, (total_kv, d))
        self._check_tensor("cu_seqlens_kv", cu_seqlens_kv, torch.int32, (R + 1,))
        self._check_tensor("cu_cand", cu_cand, torch.int32, (R + 1,))
        if O is None:
            O = torch.empty((total_cand, q, d), dtype=dt, device=Z.device)
        self._check_tensor("O", O, dt, (total_cand, q, d))
        _check(lib().xattn_forward_noalloc(self._h, _ptr(Z), _ptr(W_Q), _ptr(K), _ptr(V),
                                           _ptr(cu_seqlens_kv), _ptr(cu_cand), R, total_cand,
                                           total_kv, heads, _ptr(O), _stream(Z.device, stream)))
        return O

    def forward_train(self, Z, W_Q, K, V, cu_seqlens_kv, cu_cand, heads: int, O=None,
                      lse=None, workspace=None, stream=None, cand_kv_len=None):
        """(O, lse): forward() that also keeps each row's base-2 log softmax
        normaliser per head, lse [total_cand, q, heads] fp32, for
        backward(..., O=O, lse=lse) (include/xattn.h, xattn_forward_train)."""
        d, q, dt = self.d_model, self.q, self.torch_dtype
        total_cand, total_kv = Z.shape[0], K.shape[0]
        R = cu_seqlens_kv.numel() - 1
        self._check_tensor("Z", Z, dt, (total_cand, q, d))
        self._check_tensor("W_Q", W_Q, dt, (q, d, d))
        self._check_tensor("K", K, dt, (total_kv, d))
        if V is not None:
            self._check_tensor("V", V, dt, (total_kv, d))
        self._check_tensor("cu_seqlens_kv", cu_seqlens_kv, torch.int32, (R + 1,))
        self._check_tensor("cu_cand", cu_cand, torch.int32, (R + 1,))
        if cand_kv_len is not None:
            self._check_tensor("cand_kv_len", cand_kv_len, torch.int32, (total_cand,))
        if O is None:
            O = torch.empty((total_cand, q, d), dtype=dt, device=Z.device)
        if lse is None:
            lse = torch.empty((total_cand, q, heads), dtype=torch.float32, device=Z.device)
        self._check_tensor("O", O, dt, (total_cand, q, d))
        self._check_tensor("lse", lse, torch.float32, (total_cand, q, heads))
        if workspace is None:
            workspace = self.alloc_workspace(R, total_cand, heads)
        _check(lib().xattn_forward_train(
            self._h, _ptr(Z), _ptr(W_Q), _ptr(K), _ptr(V), _ptr(cu_seqlens_kv), _ptr(cu_cand),
            _ptr(cand_kv_len), R, total_cand, total_kv, heads, _ptr(O), _ptr(lse),
            _ptr(workspace), workspace.numel(), _stream(Z.device, stream)))
        return O, lse

    def attend(self, Z, W_Q, K, V, cu_seqlens_kv, cu_cand, heads: int, workspace, O=None,
               stream=None) -> torch.Tensor:
        """Projection + attention, reusing the plan a previous forward()/plan() of
        the same batch left in `workspace`."""
        return self.forward(Z, W_Q, K, V, cu_seqlens_kv, cu_cand, heads, O=O,
                            workspace=workspace, stream=stream, plan=False)

    def attend_q(self, Q, K, V, cu_seqlens_kv, cu_cand, heads: int, workspace, O=None,
                 stream=None, cand_kv_len=None, bind: bool = False) -> torch.Tensor:
        """Attention kernel alone over already-projected queries Q [total_cand, q, d],
        reusing the plan in `workspace`; cand_kv_len as for forward()
        (xattn_attend_q_prefix).  bind=True returns the checked call as a
        BoundCall instead of running it."""
        d, q, dt = self.d_model, self.q, self.torch_dtype
        total_cand, total_kv = Q.shape[0], K.shape[0]
        R = cu_seqlens_kv.numel() - 1
        self._check_tensor("Q", Q, dt, (total_cand, q, d))
        self._check_tensor("K", K, dt, (total_kv, d))
        if V is not None:
            self._check_tensor("V", V, dt, (total_kv, d))
        self._check_tensor("cu_seqlens_kv", cu_seqlens_kv, torch.int32, (R + 1,))
        self._check_tensor("cu_cand", cu_cand, torch.int32, (R + 1,))
        if O is None:
            O = torch.empty((total_cand, q, d), dtype=dt, device=Q.device)
        self._check_tensor("O", O, dt, (total_cand, q, d))
        if cand_kv_len is not None:
            self._check_tensor("cand_kv_len", cand_kv_len, torch.int32, (total_cand,))
            b = _call(lib().xattn_attend_q_prefix,
                      (self._h, _ptr(Q), _ptr(K), _ptr(V), _ptr(cu_seqlens_kv), _ptr(cu_cand),
                       _ptr(cand_kv_len), R, total_cand, total_kv, heads, _ptr(O),
                       _ptr(workspace), workspace.numel(), _stream(Q.device, stream)), bind)
            return b if bind else O
        b = _call(lib().xattn_attend_q,
                  (self._h, _ptr(Q), _ptr(K), _ptr(V), _ptr(cu_seqlens_kv), _ptr(cu_cand), R,
                   total_cand, total_kv, heads, _ptr(O), _ptr(workspace), workspace.numel(),
                   _stream(Q.device, stream)), bind)
        return b if bind else O

    def backward_workspace_size(self, num_requests: int, total_cand: int, total_kv: int,
                                heads: int) -> int:
        return int(lib().xattn_backward_workspace_size(self._h, num_requests, total_cand,
                                                       total_kv, heads))

    def backward(self, Z, W_Q, K, V, dO, cu_seqlens_kv, cu_cand, heads: int, workspace=None,
                 out=None, stream=None, cand_kv_len=None, O=None, lse=None) -> dict:
        """Gradients of <dO, O> for O = forward(Z, W_Q, K, V, ...) (see
        include/xattn.h, xattn_backward): returns {"dZ", "dW_Q" (fp32), "dK"
        (dH in shared mode), "dV" (None in shared mode)}; `out` may supply
        those tensors.  cand_kv_len: the per-candidate prefix of
        forward(..., cand_kv_len=...).  O and lse: the outputs of
        forward_train() on the same inputs, which replace the recomputed
        forward statistics (xattn_backward_saved)."""
        d, q, dt = self.d_model, self.q, self.torch_dtype
        total_cand, total_kv = Z.shape[0], K.shape[0]
        R = cu_seqlens_kv.numel() - 1
        self._check_tensor("Z", Z, dt, (total_cand, q, d))
        self._check_tensor("W_Q", W_Q, dt, (q, d, d))
        self._check_tensor("K", K, dt, (total_kv, d))
        if V is not None:
            self._check_tensor("V", V, dt, (total_kv, d))
        self._check_tensor("dO", dO, dt, (total_cand, q, d))
        self._check_tensor("cu_seqlens_kv", cu_seqlens_kv, torch.int32, (R + 1,))
        self._check_tensor("cu_cand", cu_cand, torch.int32, (R + 1,))
        if cand_kv_len is not None:
            self._check_tensor("cand_kv_len", cand_kv_len, torch.int32, (total_cand,))
        out = dict(out or {})
        dev = Z.device
        if out.get("dZ") is None:
            out["dZ"] = torch.empty((total_cand, q, d), dtype=dt, device=dev)
        if out.get("dW_Q") is None:
            out["dW_Q"] = torch.empty((q, d, d), dtype=torch.float32, device=dev)
        if out.get("dK") is None:
            out["dK"] = torch.empty((total_kv, d), dtype=dt, device=dev)
        if V is not None and out.get("dV") is None:
            out["dV"] = torch.empty((total_kv, d), dtype=dt, device=dev)
        if V is None:
            out["dV"] = None
        self._check_tensor("dZ", out["dZ"], dt, (total_cand, q, d))
        self._check_tensor("dW_Q", out["dW_Q"], torch.float32, (q, d, d))
        self._check_tensor("dK", out["dK"], dt, (total_kv, d))
        if V is not None:
            self._check_tensor("dV", out["dV"], dt, (total_kv, d))
        if workspace is None:
            n = self.backward_workspace_size(R, total_cand, total_kv, heads)
            workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        if O is not None or lse is not None:
            if O is None or lse is None:
                raise ValueError("the stored statistics need both O and lse")
            self._check_tensor("O", O, dt, (total_cand, q, d))
            self._check_tensor("lse", lse, torch.float32, (total_cand, q, heads))
            _check(lib().xattn_backward_saved(
                self._h, _ptr(Z), _ptr(W_Q), _ptr(K), _ptr(V), _ptr(dO), _ptr(O), _ptr(lse),
                _ptr(cu_seqlens_kv), _ptr(cu_cand), _ptr(cand_kv_len), R, total_cand, total_kv,
                heads, _ptr(out["dZ"]), _ptr(out["dW_Q"]), _ptr(out["dK"]), _ptr(out["dV"]),
                _ptr(workspace), workspace.numel(), _stream(dev, stream)))
            return out
        _check(lib().xattn_backward(self._h, _ptr(Z), _ptr(W_Q), _ptr(K), _ptr(V), _ptr(dO),
                                    _ptr(cu_seqlens_kv), _ptr(cu_cand), _ptr(cand_kv_len), R,
                                    total_cand, total_kv, heads, _ptr(out["dZ"]), _ptr(out["dW_Q"]), _ptr(out["dK"]),
                                    _ptr(out["dV"]), _ptr(workspace), workspace.numel(),
                                    _stream(dev, stream)))
        return out

    # -- coded memory ----------------------------------------------------------
    def codec_encode(self, cb: "Codebook", X, stream=None):
        """Codes [heads, n, words] uint32 and norms [heads, n] fp32 of rows X [n, d]."""
        n = X.shape[0]
        self._check_tensor("X", X, self.torch_dtype, (n, self.d_model))
        codes = torch.empty((cb.heads, n, cb.words), dtype=torch.int32, device=X.device)
        norms = torch.empty((cb.heads, n), dtype=torch.float32, device=X.device)
        s = cb.struct()
        _check(lib().xattn_codec_encode(self._h, ctypes.byref(s), cb.heads, _ptr(X), n,
                                        _ptr(codes), _ptr(norms), _stream(X.device, stream)))
        return codes, norms

    def codec_fold(self, cb_k: "Codebook", W_Q, stream=None):
        """Query weights in the keys' rotated basis (xattn_codec_fold_query_weights)."""
        self._check_tensor("W_Q", W_Q, self.torch_dtype, (self.q, self.d_model, self.d_model))
        out = torch.empty_like(W_Q)
        s = cb_k.struct()
        _check(lib().xattn_codec_fold_query_weights(self._h, ctypes.byref(s), cb_k.heads,
                                                    _ptr(W_Q), _ptr(out),
                                                    _stream(W_Q.device, stream)))
        return out

    def forward_codec(self, cb_k: "Codebook", cb_v, Z, W_Q_rot, k_codes, k_norms, v_codes,
                      v_norms, cu_seqlens_kv, cu_cand, heads: int, O=None, workspace=None,
                      stream=None, decode: bool = True) -> torch.Tensor:
        """Cross-attention over a coded memory (xattn_forward_codec).  Without a
        workspace one is allocated: with room for the decoded memory when
        `decode` (the memory decoded once per call), else the plain forward's
        (each memory tile reconstructed in LDS)."""
        d, q, dt = self.d_model, self.q, self.torch_dtype
        total_cand = Z.shape[0]
        total_kv = k_norms.shape[1]
        R = cu_seqlens_kv.numel() - 1
        self._check_tensor("Z", Z, dt, (total_cand, q, d))
        self._check_tensor("W_Q_rot", W_Q_rot, dt, (q, d, d))
        self._check_tensor("k_codes", k_codes, torch.int32, (cb_k.heads, total_kv, cb_k.words))
        self._check_tensor("k_norms", k_norms, torch.float32, (cb_k.heads, total_kv))
        if O is None:
            O = torch.empty((total_cand, q, d), dtype=dt, device=Z.device)
        if workspace is None:
            if decode:
                n = self.codec_workspace_size(R, total_cand, total_kv, heads)
                workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=Z.device)
            else:
                workspace = self.alloc_workspace(R, total_cand, heads)
        sk = cb_k.struct()
        sv = cb_v.struct() if cb_v is not None else None
        _check(lib().xattn_forward_codec(
            self._h, ctypes.byref(sk), ctypes.byref(sv) if sv is not None else None, _ptr(Z),
            _ptr(W_Q_rot), _ptr(k_codes), _ptr(k_norms), _ptr(v_codes), _ptr(v_norms),
            _ptr(cu_seqlens_kv), _ptr(cu_cand), R, total_cand, total_kv, heads, _ptr(O),
            _ptr(workspace), workspace.numel(), _stream(Z.device, stream)))
        return O

    def plan(self, cu_seqlens_kv, cu_cand, heads: int, total_cand: int, total_kv: int,
             with_row_req: bool = True, workspace=None, stream=None):
        """Integer varlen plan: returns (cu_q, row_req, tiles[n,4], tile_m) as device
        tensors (tiles sliced to the device-reported count; this reads one int)."""
        R = cu_seqlens_kv.numel() - 1
        dev = cu_cand.device
        cu_q = torch.empty(R + 1, dtype=torch.int32, device=dev)
        row_req = (torch.empty(max(total_cand * self.q, 1), dtype=torch.int32, device=dev)
                   if with_row_req else None)
        mt = max(self.max_tiles(R, total_cand, heads), 1)
        tiles = torch.empty((mt, 4), dtype=torch.int32, device=dev)
        n_tiles = torch.zeros(1, dtype=torch.int32, device=dev)
        if workspace is None:
            workspace = self.alloc_workspace(R, total_cand, heads)
        tm = ctypes.c_int32(0)
        _check(lib().xattn_plan(self._h, _ptr(cu_seqlens_kv), _ptr(cu_cand), R, total_cand,
                                total_kv, heads, _ptr(cu_q), _ptr(row_req), _ptr(tiles),
                                _ptr(n_tiles), ctypes.byref(tm), _ptr(workspace),
                                workspace.numel(), _stream(dev, stream)))
        n = int(n_tiles.item())
        rr = row_req[: total_cand * self.q] if row_req is not None else None
        return cu_q, rr, tiles[:n], tm.value

    def project(self, Z, W_Q, Q=None, stream=None, bind: bool = False) -> torch.Tensor:
        """TSP projection alone: Q[row] = Z[row] . W_Q[row % q] (output-major W_Q).
        bind=True returns the checked call as a BoundCall (Q must be given)."""
        d, q, dt = self.d_model, self.q, self.torch_dtype
        total_cand = Z.shape[0]
        self._check_tensor("Z", Z, dt, (total_cand, q, d))
        self._check_tensor("W_Q", W_Q, dt, (q, d, d))
        if bind and Q is None:
            raise ValueError("a bound call needs Q")
        if Q is None:
            Q = torch.empty((total_cand, q, d), dtype=dt, device=Z.device)
        self._check_tensor("Q", Q, dt, (total_cand, q, d))
        b = _call(lib().xattn_project,
                  (self._h, _ptr(Z), _ptr(W_Q), total_cand, _ptr(Q), _stream(Z.device, stream)),
                  bind)
        return b if bind else Q

    def output(self, Z, W_go, O, W_o, workspace, Y=None, stream=None) -> torch.Tensor:
        """Output gate and projection of Eq. (7):
        Y[row] = (O[row] * sigmoid(Z[row] . W_go[row % q])) . W_o (output-major
        weights); uses the end of `workspace` as scratch (see include/xattn.h)."""
        d, q, dt = self.d_model, self.q, self.torch_dtype
        total_cand = Z.shape[0]
        self._check_tensor("Z", Z, dt, (total_cand, q, d))
        self._check_tensor("W_go", W_go, dt, (q, d, d))
        self._check_tensor("O", O, dt, (total_cand, q, d))
        self._check_tensor("W_o", W_o, dt, (d, d))
        if Y is None:
            Y = torch.empty((total_cand, q, d), dtype=dt, device=Z.device)
        self._check_tensor("Y", Y, dt, (total_cand, q, d))
        _check(lib().xattn_output(self._h, _ptr(Z), _ptr(W_go), _ptr(O), _ptr(W_o), total_cand,
                                  _ptr(Y), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(Z.device, stream)))
        return Y

    def device_error(self, workspace, stream=None) -> int:
        """Synchronise and read the device-side offset-validation flag (0: the
        offsets were consistent; else 1 = cu_seqlens_kv, 2 = cu_cand).  The C
        call reports a set flag as XATTN_EDEVICE_VALIDATION; here the flag is
        returned either way."""
        flag = ctypes.c_int32(0)
        st = lib().xattn_device_error(self._h, _ptr(workspace), ctypes.byref(flag),
                                      _stream(workspace.device, stream))
        if st not in (XATTN_OK, XATTN_EDEVICE_VALIDATION):
            _check(st)
        return flag.value


def to_device(wl, device="cuda"):
    """Upload a workloads.Workload's arrays (already exactly representable in the
    workload's dtype) as device tensors: dict of Z, W_Q, K, V, cu_kv, cu_cand."""
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

    def up(a):
        return None if a is None else torch.from_numpy(a).to(device).to(dt).contiguous()
    return {
        "Z": up(wl.Z), "W_Q": up(wl.wt), "K": up(wl.K), "V": up(wl.V),
        "cu_kv": torch.from_numpy(wl.cu_kv).to(device), "cu_cand": torch.from_numpy(wl.cu_cand).to(device),
    }
