"""Python binding of libstatekv, the StateKV frame step for AMD MI355X (gfx950).

Argument marshalling only: every step of the frame step runs in the HIP
kernels of libstatekv.so behind the C ABI of include/statekv.h.  PyTorch
provides device memory and the HIP stream.  There is no fallback: if the
library cannot be loaded, or no GPU is visible, the calls raise.

Method: paper note "Linear Scaling Video VLMs for Long Video Understanding"
(papernotes.org, ECCV 2026), section 方法详解 (关键设计 1-3).
"""
from __future__ import annotations

import ctypes
import os
import re

import torch  # noqa: F401  (loads the HIP runtime that the library links to)

from ._build import build as build_library
from ._build import library_path

STATEKV_OK = 0
STATEKV_EINVAL = -1
STATEKV_EORDER = -2
STATEKV_ECAPACITY = -3
STATEKV_ENOMEM = -4
STATEKV_EDEVICE = -5
STATEKV_ENONFINITE = -6
STATEKV_ESCRATCH = -7
STATIC_SCRATCH_BYTES = 32 << 20

DTYPE_BF16 = 1
DTYPE_F32 = 2

FLAG_ALWAYS_SCORE = 1
FLAG_KERNEL_TIMING = 2
FLAG_RECENT_WINDOW = 4

KERNEL_NAMES = ["rope_select", "attn_fwd", "score_merge", "select_view",
                "decode_rope", "decode_attn", "decode_merge"]

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "statekv.h")


class LayerCfg(ctypes.Structure):
    _fields_ = [
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("tokens_per_frame", ctypes.c_int32),
        ("max_frames", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("rope_base", ctypes.c_double),
        ("rope_orig_ctx", ctypes.c_int32),
        ("max_text", ctypes.c_int32),
        ("n_layers", ctypes.c_int32),
    ]


class View(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("pos", ctypes.c_void_p),
        ("count", ctypes.c_int64),
        ("head_stride", ctypes.c_int64),
        ("token_stride", ctypes.c_int64),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("frames_done", ctypes.c_int32),
        ("n_layers", ctypes.c_int32),
        ("layer_stride", ctypes.c_int64),
        ("pos_layer_stride", ctypes.c_int64),
    ]


class ScoresView(ctypes.Structure):
    _fields_ = [
        ("scores", ctypes.c_void_p),
        ("pool_pos", ctypes.c_void_p),
        ("keep_flag", ctypes.c_void_p),
        ("pool", ctypes.c_int32),
        ("kept", ctypes.c_int32),
        ("frame", ctypes.c_int32),
        ("n_layers", ctypes.c_int32),
        ("layer_stride", ctypes.c_int64),
    ]


class StateKVError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {error_string(code)} ({code})")


_lib = None
_hip = None


def declared_functions() -> list:
    """Names of the functions include/statekv.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(statekv_[a-z_]+)\s*\(", text)))


def load_library(build_if_missing: bool = True) -> ctypes.CDLL:
    """Load libstatekv.so (building it first if it does not exist)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        if not build_if_missing:
            raise RuntimeError(f"{path} is not built")
        build_library()
    lib = ctypes.CDLL(path)
    P, I32, U32, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float
    lib.statekv_create.argtypes = [ctypes.POINTER(LayerCfg), I32, F32, ctypes.POINTER(P)]
    lib.statekv_set_stream.argtypes = [P, P]
    lib.statekv_prefill_frame.argtypes = [P, P, P, P, I32, P]
    lib.statekv_prefill_frame_static.argtypes = [P, P, P, P, I32, P]
    lib.statekv_decode.argtypes = [P, P, P, P, I32, P]
    lib.statekv_compressed_view.argtypes = [P, ctypes.POINTER(View)]
    lib.statekv_detailed_view.argtypes = [P, ctypes.POINTER(View)]
    lib.statekv_scores.argtypes = [P, ctypes.POINTER(ScoresView)]
    lib.statekv_set_flags.argtypes = [P, U32]
    lib.statekv_kernel_times.argtypes = [P, ctypes.POINTER(F32), ctypes.POINTER(I32), I32, I32]
    lib.statekv_destroy.argtypes = [P]
    lib.statekv_destroy.restype = None
    lib.statekv_strerror.argtypes = [ctypes.c_int]
    lib.statekv_strerror.restype = ctypes.c_char_p
    for name in ("statekv_create", "statekv_set_stream", "statekv_prefill_frame",
                 "statekv_prefill_frame_static", "statekv_decode",
                 "statekv_compressed_view", "statekv_detailed_view", "statekv_scores",
                 "statekv_set_flags", "statekv_kernel_times"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def error_string(code: int) -> str:
    return load_library().statekv_strerror(code).decode()


def _hip_runtime() -> ctypes.CDLL:
    """The HIP runtime already loaded by torch (same SONAME as the library's)."""
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so.7")
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _hip.hipMemcpy.restype = ctypes.c_int
    return _hip


def _copy_to_tensor(ptr: int, shape, dtype: torch.dtype, device) -> torch.Tensor:
    out = torch.empty(shape, dtype=dtype, device=device)
    nbytes = out.numel() * out.element_size()
    if nbytes:
        rc = _hip_runtime().hipMemcpy(out.data_ptr(), ptr, nbytes, 3)  # device to device
        if rc != 0:
            raise RuntimeError(f"hipMemcpy failed ({rc})")
    return out


_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}
_ABI_DTYPE = {"bf16": DTYPE_BF16, "f32": DTYPE_F32}


class StateKV:
    """One layer's StateKV state on the current GPU (compressed state C and detailed cache D),
    or with n_layers > 1 a stack of independent layers stepped together: frame tensors then
    carry a leading layer dimension ([L][T][H][d]) and views take a layer index."""

    def __init__(self, *, n_q_heads: int, n_kv_heads: int, head_dim: int,
                 tokens_per_frame: int, max_frames: int, budget: int, alpha: float = 1.0,
                 dtype: str = "bf16", rope_base: float = 1e6, rope_orig_ctx: int = 32768,
                 max_text: int = 0, n_layers: int = 1, stream=None):
        self._lib = load_library()
        if dtype not in _ABI_DTYPE:
            raise ValueError(f"dtype must be 'bf16' or 'f32', not {dtype!r}")
        self.dtype = dtype
        self.torch_dtype = _TORCH_DTYPE[dtype]
        self.Hq, self.Hkv, self.d = n_q_heads, n_kv_heads, head_dim
        self.T, self.max_frames, self.budget = tokens_per_frame, max_frames, budget
        self.alpha = alpha
        self.max_text = max_text
        self.L = n_layers
        self.device = torch.device("cuda", torch.cuda.current_device())
        cfg = LayerCfg(n_q_heads, n_kv_heads, head_dim, tokens_per_frame, max_frames,
                       _ABI_DTYPE[dtype], float(rope_base), rope_orig_ctx, max_text, n_layers)
        handle = ctypes.c_void_p()
        rc = self._lib.statekv_create(ctypes.byref(cfg), budget, float(alpha), ctypes.byref(handle))
        if rc != STATEKV_OK:
            raise StateKVError(rc, "statekv_create")
        self._h = handle
        self.set_stream(stream if stream is not None else torch.cuda.current_stream())

    # -- lifetime -----------------------------------------------------------
    def close(self):
        if getattr(self, "_h", None):
            self._lib.statekv_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, rc: int, what: str):
        if rc != STATEKV_OK:
            raise StateKVError(rc, what)

    # -- configuration --------------------------------------------------------
    def set_stream(self, stream):
        self.stream = stream
        self._check(self._lib.statekv_set_stream(self._h, ctypes.c_void_p(stream.cuda_stream)),
                    "statekv_set_stream")

    def set_flags(self, flags: int):
        self._check(self._lib.statekv_set_flags(self._h, flags), "statekv_set_flags")

    # -- stream ordering ------------------------------------------------------
    def _launch(self, fn, tensors):
        """Run a library call on the state's stream, ordered after the work queued
        on torch's current stream (which produced the inputs); the current stream
        then waits for the call, so its output is ready there, and the tensors are
        recorded on the state's stream for the caching allocator."""
        cur = torch.cuda.current_stream(self.device)
        if cur == self.stream:
            fn()
            return
        self.stream.wait_stream(cur)
        fn()
        cur.wait_stream(self.stream)
        for t in tensors:
            t.record_stream(self.stream)

    # -- the frame step -------------------------------------------------------
    def _shape(self, tokens: int, heads: int):
        one = (tokens, heads, self.d)
        return one if self.L == 1 else (self.L,) + one

    def _frame_tensor(self, x: torch.Tensor, heads: int, name: str, tokens=None):
        want = self._shape(self.T if tokens is None else tokens, heads)
        if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
            raise ValueError(f"{name} must be a CUDA/HIP tensor")
        if x.dtype != self.torch_dtype or tuple(x.shape) != want or not x.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {self.torch_dtype} tensor of shape {want}")

    def prefill_frame(self, Q, K, V, n: int, out=None) -> torch.Tensor:
        """Run frame n; returns O [T][Hq][d] ([L][T][Hq][d] for a stack), written
        asynchronously on the state's stream.  When torch's current stream is not
        the state's, the step is ordered after it and it waits for the step."""
        self._frame_tensor(Q, self.Hq, "Q")
        self._frame_tensor(K, self.Hkv, "K")
        self._frame_tensor(V, self.Hkv, "V")
        if out is None:
            out = torch.empty(self._shape(self.T, self.Hq), dtype=self.torch_dtype, device=Q.device)
        else:
            self._frame_tensor(out, self.Hq, "out")
        self._launch(lambda: self._check(
            self._lib.statekv_prefill_frame(self._h, Q.data_ptr(), K.data_ptr(), V.data_ptr(), n,
                                            out.data_ptr()),
            "statekv_prefill_frame"), (Q, K, V, out))
        return out

    # -- the text phase ---------------------------------------------------------
    def decode(self, Q, K, V, out=None) -> torch.Tensor:
        """Append t text tokens (Q [t][Hq][d], K, V [t][Hkv][d]) after everything
        processed so far and attend them over the whole detailed cache; returns
        O [t][Hq][d] (asynchronous on the state's stream).  A stack takes and returns
        [L][t][H][d]."""
        rank = 3 if self.L == 1 else 4
        t = Q.shape[rank - 3] if isinstance(Q, torch.Tensor) and Q.dim() == rank else -1
        self._frame_tensor(Q, self.Hq, "Q", t)
        self._frame_tensor(K, self.Hkv, "K", t)
        self._frame_tensor(V, self.Hkv, "V", t)
        if out is None:
            out = torch.empty(self._shape(t, self.Hq), dtype=self.torch_dtype, device=Q.device)
        else:
            self._frame_tensor(out, self.Hq, "out", t)
        self._launch(lambda: self._check(
            self._lib.statekv_decode(self._h, Q.data_ptr(), K.data_ptr(), V.data_ptr(), t,
                                     out.data_ptr()),
            "statekv_decode"), (Q, K, V, out))
        return out

    # -- views (copied into new tensors) ------------------------------------------
    def _layer(self, layer: int) -> int:
        if not 0 <= layer < self.L:
            raise ValueError(f"layer {layer} out of range for a stack of {self.L}")
        return layer

    def compressed_view(self, layer: int = 0):
        """(Kbar [Hkv][count][d], Vbar [Hkv][count][d], pos [count] int32) of one layer,
        copies in slot order."""
        self._layer(layer)
        v = View()
        self._check(self._lib.statekv_compressed_view(self._h, ctypes.byref(v)),
                    "statekv_compressed_view")
        cap = v.head_stride // v.head_dim
        esz = 2 if self.dtype == "bf16" else 4
        ko = layer * v.layer_stride * esz
        k = _copy_to_tensor(v.k + ko, (v.n_kv_heads, cap, v.head_dim), self.torch_dtype, self.device)
        vv = _copy_to_tensor(v.v + ko, (v.n_kv_heads, cap, v.head_dim), self.torch_dtype, self.device)
        pos = _copy_to_tensor(v.pos + layer * v.pos_layer_stride * 4, (v.count,), torch.int32,
                              self.device)
        return k[:, : v.count].contiguous(), vv[:, : v.count].contiguous(), pos

    def detailed_view(self, layer: int = 0):
        """(D_K [count][Hkv][d], D_V [count][Hkv][d]) of one layer, copies;
        count = n*T + text tokens."""
        self._layer(layer)
        v = View()
        self._check(self._lib.statekv_detailed_view(self._h, ctypes.byref(v)),
                    "statekv_detailed_view")
        shape = (v.count, v.n_kv_heads, v.head_dim)
        ko = layer * v.layer_stride * (2 if self.dtype == "bf16" else 4)
        return (_copy_to_tensor(v.k + ko, shape, self.torch_dtype, self.device),
                _copy_to_tensor(v.v + ko, shape, self.torch_dtype, self.device))

    def scores(self, layer: int = 0):
        """dict(frame, scores [pool] f32, pool_pos [pool] i32, keep_flag [pool] i32) of one
        layer, or None."""
        self._layer(layer)
        sv = ScoresView()
        self._check(self._lib.statekv_scores(self._h, ctypes.byref(sv)), "statekv_scores")
        if sv.frame < 0:
            return None
        o = layer * sv.layer_stride * 4
        return {
            "frame": sv.frame,
            "scores": _copy_to_tensor(sv.scores + o, (sv.pool,), torch.float32, self.device),
            "pool_pos": _copy_to_tensor(sv.pool_pos + o, (sv.pool,), torch.int32, self.device),
            "keep_flag": _copy_to_tensor(sv.keep_flag + o, (sv.pool,), torch.int32, self.device),
        }

    def kernel_times(self, reset: bool = False):
        """{kernel name: (total ms, launches)} since the last reset (needs FLAG_KERNEL_TIMING)."""
        n = len(KERNEL_NAMES)
        ms = (ctypes.c_float * n)()
        cnt = (ctypes.c_int32 * n)()
        self._check(self._lib.statekv_kernel_times(self._h, ms, cnt, n, int(reset)),
                    "statekv_kernel_times")
        return {name: (ms[i], cnt[i]) for i, name in enumerate(KERNEL_NAMES)}


__all__ = ["StateKV", "StateKVError", "load_library", "build_library", "library_path",
           "declared_functions", "error_string", "KERNEL_NAMES",
           "FLAG_ALWAYS_SCORE", "FLAG_KERNEL_TIMING", "FLAG_RECENT_WINDOW"]
