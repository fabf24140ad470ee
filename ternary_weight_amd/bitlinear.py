"""Python binding of libbitlinear.so (the C ABI declared in include/bitlinear.h).

Argument marshalling only: torch tensors are checked for dtype, device and
layout and passed as raw device pointers with the current HIP stream; every
step of the path runs in the library's HIP kernels (or, for ``i2s_pack``, in
its host C++).  Importing this module raises ImportError when the library has
not been built: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitlinear.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m ternary_weight_amd.build`")

# Load torch first when it is installed: it carries its own HIP runtime, and
# the library must bind to that same runtime (loaded first, the library would
# pull in the system one, and torch's tensors would then belong to another
# runtime than the library's kernel launches).
try:
    import torch as _torch_first  # noqa: F401
except ImportError:
    pass

_lib = ctypes.CDLL(LIB_PATH)

BL_OK = 0
BL_ERR_INVALID_ARGUMENT = -1
BL_ERR_UNSUPPORTED = -2
BL_ERR_MISALIGNED = -3
BL_ERR_NONFINITE = -4
BL_ERR_HIP = -5
BL_ERR_NOMEM = -6
BL_ERR_INTERNAL = -7
BL_ERR_NOT_FOUND = -8

_p, _i64, _f32, _i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int32

# BL_LAUNCH_* of include/bitlinear.h
LAUNCH_KINDS = {0: "decode", 1: "prefill", 2: "quant", 3: "decode_fused", 4: "quant_shared",
                5: "quant_glue", 6: "decode_fused_glue", 7: "quant_merged"}


class BlDesc(ctypes.Structure):
    """Mirror of ``bl_desc``."""
    _fields_ = [("x", _p), ("norm_w", _p), ("packed_w", _p), ("w_scale", _f32), ("eps", _f32),
                ("M", _i64), ("K", _i64), ("N", _i64), ("y", _p), ("norm_w_f16", _i32),
                ("up", _p), ("act", _i32)]


class GgufTensor(ctypes.Structure):
    """Mirror of ``bl_gguf_tensor``."""
    _fields_ = [("type", _i32), ("n_dims", _i32), ("dims", _i64 * 4), ("offset", ctypes.c_uint64),
                ("nbytes", ctypes.c_uint64)]


_SIGS = {
    "bl_status_string": ([_i32], ctypes.c_char_p),
    "bl_k_max": ([], _i64),
    "i2s_packed_bytes": ([_i64, _i64], ctypes.c_size_t),
    "i2s_pack": ([_p, _i64, _i64, _p, ctypes.c_size_t, _p], _i32),
    "bl_gguf_find_tensor": ([_p, ctypes.c_size_t, ctypes.c_char_p, ctypes.POINTER(GgufTensor)], _i32),
    "i2s_pack_device": ([_p, _i64, _i64, _p, ctypes.c_size_t, _p, _p], _i32),
    "bitlinear_forward": ([_p, _p, _p, _f32, _i64, _i64, _i64, _f32, _p, _p], _i32),
    "bitlinear_forward_prefill_fused": ([_p, _p, _p, _f32, _i64, _i64, _i64, _f32, _p, _p], _i32),
    "bitlinear_forward_prefill_fused_nwf16": ([_p, _p, _p, _f32, _i64, _i64, _i64, _f32, _p, _p], _i32),
    "bitlinear_quant": ([_p, _p, _i64, _i64, _f32, _p, _p, _p], _i32),
    "bitlinear_matmul_i32": ([_p, _p, _i64, _i64, _i64, _p, _p], _i32),
    "bitlinear_glu_quant": ([_p, _p, _i32, _p, _i64, _i64, _f32, _p, _p, _p], _i32),
    "bitlinear_glu_forward": ([_p, _p, _i32, _p, _p, _f32, _i64, _i64, _i64, _f32, _p, _p], _i32),
    "bitlinear_forward_nwf16": ([_p, _p, _p, _f32, _i64, _i64, _i64, _f32, _p, _p], _i32),
    "bitlinear_quant_nwf16": ([_p, _p, _i64, _i64, _f32, _p, _p, _p], _i32),
    "bitlinear_glu_quant_nwf16": ([_p, _p, _i32, _p, _i64, _i64, _f32, _p, _p, _p], _i32),
    "bitlinear_glu_forward_nwf16": ([_p, _p, _i32, _p, _p, _f32, _i64, _i64, _i64, _f32, _p, _p], _i32),
    "bl_group_create": ([ctypes.POINTER(BlDesc), _i32, ctypes.POINTER(_p)], _i32),
    "bl_group_forward": ([_p, _p], _i32),
    "bl_group_quant": ([_p, _p], _i32),
    "bl_group_matmul": ([_p, _p], _i32),
    "bl_group_destroy": ([_p], _i32),
    "bl_group_matmul_launches": ([_p], _i32),
    "bl_group_matmul_launch_info": ([_p, _i32, _p, _p, _p], _i32),
    "bl_group_matmul_launch": ([_p, _i32, _p], _i32),
    "bl_group_forward_launches": ([_p], _i32),
    "bl_group_forward_launch_info": ([_p, _i32, _p, _p, _p], _i32),
    "bl_group_forward_launch": ([_p, _i32, _p], _i32),
    "bitlinear_forward_batched": ([ctypes.POINTER(BlDesc), _i32, _p], _i32),
    "bl_prefill_splits": ([ctypes.POINTER(BlDesc), _i32, _i32, ctypes.POINTER(_i32)], _i32),
    "bitlinear_forward_noalloc": ([_p, _p, _p, _f32, _i64, _i64, _i64, _f32, _p, _p], _i32),
    "bl_release_workspace": ([], _i32),
    # measurement probes (include/bitlinear_probe.h)
    "bl_probe_read": ([_p, ctypes.c_size_t, _p, _i32, _p], _i32),
    "bl_probe_copy": ([_p, _p, ctypes.c_size_t, _i32, _p], _i32),
    "bl_probe_write": ([_p, ctypes.c_size_t, _i32, _i32, _p], _i32),
    "bl_probe_mixed": ([_p, ctypes.c_size_t, _p, ctypes.c_size_t, _i32, _p, _i32, _p], _i32),
    "bl_probe_mfma_i8": ([_i32, _i32, _i32, _p, _p], _i32),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTED = tuple(_SIGS)
lib = _lib


class BitLinearError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {bl_status_string(status)} ({status})")


def bl_status_string(status: int) -> str:
    return _lib.bl_status_string(status).decode()


def _check(status: int, what: str) -> None:
    if status != BL_OK:
        raise BitLinearError(status, what)


def bl_k_max() -> int:
    return int(_lib.bl_k_max())


def i2s_packed_bytes(K: int, N: int) -> int:
    return int(_lib.i2s_packed_bytes(K, N))


def i2s_pack(w: np.ndarray) -> tuple[np.ndarray, float]:
    """Host packing: float32 [N, K] -> (uint8 I2_S buffer, scale)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be [N, K]")
    N, K = w.shape
    nbytes = i2s_packed_bytes(K, N)
    out = np.empty(max(nbytes, 1), dtype=np.uint8)
    scale = ctypes.c_float(0.0)
    _check(_lib.i2s_pack(w.ctypes.data, K, N, out.ctypes.data, nbytes, ctypes.byref(scale)),
           "i2s_pack")
    return out, float(scale.value)


GGUF_F32, GGUF_F16, GGUF_I2S = 0, 1, 36  # ggml type ids


def gguf_find_tensor(file: np.ndarray, name: str) -> dict:
    """A tensor's type, dims (innermost first), data offset and size in a GGUF
    file image (uint8 numpy array); raises BitLinearError if absent or the
    image is malformed."""
    file = np.ascontiguousarray(file, dtype=np.uint8)
    t = GgufTensor()
    _check(_lib.bl_gguf_find_tensor(file.ctypes.data, file.size, name.encode(), ctypes.byref(t)),
           f"bl_gguf_find_tensor({name})")
    return dict(type=int(t.type), dims=[int(t.dims[i]) for i in range(t.n_dims)],
                offset=int(t.offset), nbytes=int(t.nbytes))


def gguf_i2s_weight(file: np.ndarray, name: str) -> tuple[np.ndarray, float, int, int]:
    """(I2_S buffer (codes + scale, a view of the file), scale, K, N) of a
    projection weight stored in a GGUF file image."""
    t = gguf_find_tensor(file, name)
    if t["type"] != GGUF_I2S:
        raise ValueError(f"{name} has ggml type {t['type']}, not I2_S (36)")
    K, N = t["dims"]
    buf = np.asarray(file, dtype=np.uint8)[t["offset"]:t["offset"] + t["nbytes"]]
    return buf, float(buf[-4:].view(np.float32)[0]), K, N


# ---------------------------------------------------------------- device ---

# torch and the few of its entry points the hot path uses, bound once: a
# small projection's call is a few microseconds of GPU time, and per-call
# module lookups and Stream objects cost the host as much.
_TORCH = None
_TENSOR = None
_RAW_STREAM = None  # current stream's raw handle by device index, where torch offers it
_GET_DEVICE = None


def _torch():
    global _TORCH, _TENSOR, _RAW_STREAM, _GET_DEVICE
    if _TORCH is None:
        import torch
        _TENSOR = torch.Tensor
        _RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _GET_DEVICE = getattr(torch._C, "_cuda_getDevice", None)
        _TORCH = torch
    return _TORCH


def _stream_handle(stream) -> int | None:
    """The HIP stream handle: the given stream's, or the current stream's."""
    if stream is None:
        torch = _torch()
        if _RAW_STREAM is not None and _GET_DEVICE is not None:
            return _RAW_STREAM(_GET_DEVICE())
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t, dtype, name: str, shape=None) -> int:
    """t's device pointer after checking that t is a contiguous GPU tensor of
    dtype (and shape); one combined test on the common path, the specific
    error otherwise."""
    if _TENSOR is None:
        _torch()
    if (isinstance(t, _TENSOR) and t.is_cuda and t.dtype is dtype and t.is_contiguous()
            and (shape is None or t.shape == shape)):
        return t.data_ptr()
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _norm(norm_w, K):
    """The norm weight's pointer (None: no per-projection norm) and whether it
    is float16 (the pages' stored dtype for norms) rather than float32."""
    torch = _torch()
    if norm_w is None:
        return None, False
    f16 = norm_w.dtype == torch.float16
    return _dev(norm_w, torch.float16 if f16 else torch.float32, "norm_w", (K,)), f16


def i2s_pack_device(w, packed=None, read_scale: bool = True, stream=None):
    """Device packing: float32 [N, K] GPU tensor -> (uint8 I2_S GPU tensor,
    scale).  read_scale False only enqueues the work (the scale is then None;
    it is the buffer's last four bytes)."""
    torch = _torch()
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    N, K = w.shape
    nbytes = i2s_packed_bytes(K, N)
    if packed is None:
        packed = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=w.device)
    scale = ctypes.c_float(0.0)
    _check(_lib.i2s_pack_device(
        _dev(w, torch.float32, "w"), K, N, _dev(packed, torch.uint8, "packed"), packed.numel(),
        ctypes.byref(scale) if read_scale else None, _stream_handle(stream)), "i2s_pack_device")
    return packed, (float(scale.value) if read_scale else None)


def bitlinear_forward(x, norm_w, packed_w, w_scale: float, N: int, eps: float, y=None,
                      stream=None):
    """y[M, N] (float32) = BitLinear(x[M, K]) on the GPU; returns y."""
    torch = _torch()
    M, K = x.shape
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    nw, f16 = _norm(norm_w, K)
    fn = _lib.bitlinear_forward_nwf16 if f16 else _lib.bitlinear_forward
    _check(fn(
        _dev(x, torch.float32, "x"), nw,
        _dev(packed_w, torch.uint8, "packed_w"), w_scale, M, K, N, eps,
        _dev(y, torch.float32, "y", (M, N)), _stream_handle(stream)), "bitlinear_forward")
    return y


def bitlinear_forward_prefill_fused(x, norm_w, packed_w, w_scale: float, N: int, eps: float, y=None,
                                    stream=None):
    """bitlinear_forward with the quantization inside the prefill product's
    producer (same results); returns y."""
    torch = _torch()
    M, K = x.shape
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    nw, f16 = _norm(norm_w, K)
    fn = _lib.bitlinear_forward_prefill_fused_nwf16 if f16 else _lib.bitlinear_forward_prefill_fused
    _check(fn(
        _dev(x, torch.float32, "x"), nw,
        _dev(packed_w, torch.uint8, "packed_w"), w_scale, M, K, N, eps,
        _dev(y, torch.float32, "y", (M, N)), _stream_handle(stream)), "bitlinear_forward_prefill_fused")
    return y


def bitlinear_forward_noalloc(x, norm_w, packed_w, w_scale: float, N: int, eps: float, y,
                              stream=None):
    """bitlinear_forward with the library's static device scratch instead of
    its allocated workspace (y must be given: nothing is allocated)."""
    torch = _torch()
    M, K = x.shape
    nw = None if norm_w is None else _dev(norm_w, torch.float32, "norm_w", (K,))
    _check(_lib.bitlinear_forward_noalloc(
        _dev(x, torch.float32, "x"), nw, _dev(packed_w, torch.uint8, "packed_w"), w_scale, M, K, N,
        eps, _dev(y, torch.float32, "y", (M, N)), _stream_handle(stream)), "bitlinear_forward_noalloc")
    return y


def bitlinear_quant(x, norm_w, eps: float, xq=None, x_factor=None, stream=None):
    """(int8 codes [M, K], float32 factor [M]) of the fused RMSNorm + quant kernel."""
    torch = _torch()
    M, K = x.shape
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if x_factor is None:
        x_factor = torch.empty((M,), dtype=torch.float32, device=x.device)
    nw, f16 = _norm(norm_w, K)
    fn = _lib.bitlinear_quant_nwf16 if f16 else _lib.bitlinear_quant
    _check(fn(
        _dev(x, torch.float32, "x"), nw, M, K, eps,
        _dev(xq, torch.int8, "xq", (M, K)), _dev(x_factor, torch.float32, "x_factor", (M,)),
        _stream_handle(stream)), "bitlinear_quant")
    return xq, x_factor


def bitlinear_matmul_i32(xq, packed_w, N: int, acc=None, stream=None):
    """Exact int32 [M, N] product of int8 codes with the ternary weights."""
    torch = _torch()
    M, K = xq.shape
    if acc is None:
        acc = torch.empty((M, N), dtype=torch.int32, device=xq.device)
    _check(_lib.bitlinear_matmul_i32(
        _dev(xq, torch.int8, "xq"), _dev(packed_w, torch.uint8, "packed_w"), M, K, N,
        _dev(acc, torch.int32, "acc", (M, N)), _stream_handle(stream)), "bitlinear_matmul_i32")
    return acc


def _descs(items):
    """bl_desc array of group-style item dicts (see Group)."""
    torch = _torch()
    descs = (BlDesc * len(items))()
    for i, it in enumerate(items):
        x, y = it["x"], it["y"]
        M, K = x.shape
        nw, f16 = _norm(it.get("norm_w"), K)
        up = it.get("up")
        descs[i] = BlDesc(_dev(x, torch.float32, "x"), nw,
                          _dev(it["packed_w"], torch.uint8, "packed_w"),
                          float(it["w_scale"]), float(it["eps"]), M, K, int(it["N"]),
                          _dev(y, torch.float32, "y", (M, int(it["N"]))), int(f16),
                          None if up is None else _dev(up, torch.float32, "up", (M, K)),
                          int(it.get("act", ACT_SILU)) if up is not None else 0)
    return descs


def prefill_splits(items, cus: int) -> list[int]:
    """The K split factor each item would get in a Group on a device with
    `cus` compute units (1: not split); see bl_prefill_splits."""
    descs = _descs(items)
    out = (_i32 * len(items))()
    _check(_lib.bl_prefill_splits(descs, len(items), int(cus), out), "bl_prefill_splits")
    return [int(v) for v in out]


def bitlinear_forward_batched(items, stream=None) -> None:
    """Every item's forward (Group-style dicts, outputs in item["y"]) in one
    stateless call."""
    descs = _descs(items)
    _check(_lib.bitlinear_forward_batched(descs, len(items), _stream_handle(stream)),
           "bitlinear_forward_batched")


class Group:
    """Many independent projections run as one launch per stage.

    ``items`` is a sequence of dicts with keys x, norm_w, packed_w, w_scale,
    eps, N and y (torch tensors on the GPU where applicable; norm_w float32 or
    float16, None or absent: no per-projection norm), and optionally up and
    act: the FFN glue, the input is then act(x) * up with x the gate (act
    ACT_SILU or ACT_GELU_TANH).  The tensors are kept referenced for the
    group's lifetime.
    """

    def __init__(self, items):
        self._keep = list(items)
        descs = _descs(items)
        handle = _p()
        _check(_lib.bl_group_create(descs, len(items), ctypes.byref(handle)), "bl_group_create")
        self._h = handle

    def forward(self, stream=None) -> None:
        _check(_lib.bl_group_forward(self._h, _stream_handle(stream)), "bl_group_forward")

    def quant(self, stream=None) -> None:
        _check(_lib.bl_group_quant(self._h, _stream_handle(stream)), "bl_group_quant")

    def matmul(self, stream=None) -> None:
        _check(_lib.bl_group_matmul(self._h, _stream_handle(stream)), "bl_group_matmul")

    def _launch_list(self, n_fn, info_fn, what) -> list[dict]:
        out = []
        for i in range(n_fn(self._h)):
            kind, bucket, count = _i32(), _i32(), _i32()
            _check(info_fn(self._h, i, ctypes.byref(kind), ctypes.byref(bucket), ctypes.byref(count)),
                   what)
            out.append(dict(kind=LAUNCH_KINDS[kind.value], bucket=bucket.value, count=count.value))
        return out

    def launches(self) -> list[dict]:
        """The matmul stage's launches: kind ("decode"/"prefill"), bucket, count."""
        return self._launch_list(_lib.bl_group_matmul_launches, _lib.bl_group_matmul_launch_info,
                                 "bl_group_matmul_launch_info")

    def matmul_launch(self, i: int, stream=None) -> None:
        _check(_lib.bl_group_matmul_launch(self._h, i, _stream_handle(stream)),
               "bl_group_matmul_launch")

    def forward_launches(self) -> list[dict]:
        """The forward's launches: kind ("quant"/"decode"/"prefill"), bucket, count."""
        return self._launch_list(_lib.bl_group_forward_launches, _lib.bl_group_forward_launch_info,
                                 "bl_group_forward_launch_info")

    def forward_launch(self, i: int, stream=None) -> None:
        _check(_lib.bl_group_forward_launch(self._h, i, _stream_handle(stream)),
               "bl_group_forward_launch")

    def close(self) -> None:
        if self._h:
            _check(_lib.bl_group_destroy(self._h), "bl_group_destroy")
            self._h = _p()
            self._keep = []

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            if self._h:
                _lib.bl_group_destroy(self._h)
        except Exception:
            pass


def bl_release_workspace() -> None:
    _check(_lib.bl_release_workspace(), "bl_release_workspace")


def probe_read(buf, sink, blocks: int, stream=None) -> None:
    """Streaming-read probe over a uint8 device tensor (see bitlinear_probe.h)."""
    torch = _torch()
    _check(_lib.bl_probe_read(_dev(buf, torch.uint8, "buf"), buf.numel(),
                              _dev(sink, torch.int32, "sink"), blocks, _stream_handle(stream)),
           "bl_probe_read")


def probe_copy(src, dst, blocks: int, stream=None) -> None:
    torch = _torch()
    if src.numel() != dst.numel():
        raise ValueError("src and dst sizes differ")
    _check(_lib.bl_probe_copy(_dev(src, torch.uint8, "src"), _dev(dst, torch.uint8, "dst"),
                              src.numel(), blocks, _stream_handle(stream)), "bl_probe_copy")


def probe_write(dst, blocks: int, nontemporal: bool = False, stream=None) -> None:
    """Streaming-write probe over a uint8 device tensor (see bitlinear_probe.h)."""
    torch = _torch()
    _check(_lib.bl_probe_write(_dev(dst, torch.uint8, "dst"), dst.numel(), blocks, int(nontemporal),
                               _stream_handle(stream)), "bl_probe_write")


def probe_mixed(src, dst, reads_per_write: int, sink, blocks: int, stream=None) -> None:
    """Mixed read/write probe over uint8 device tensors (see bitlinear_probe.h)."""
    torch = _torch()
    _check(_lib.bl_probe_mixed(_dev(src, torch.uint8, "src"), src.numel(), _dev(dst, torch.uint8, "dst"),
                               dst.numel(), reads_per_write, _dev(sink, torch.int32, "sink"), blocks,
                               _stream_handle(stream)), "bl_probe_mixed")


def probe_mfma_i8(iters: int, blocks: int, sink, shape: int = 16, stream=None) -> None:
    torch = _torch()
    _check(_lib.bl_probe_mfma_i8(iters, blocks, shape, _dev(sink, torch.int32, "sink"),
                                 _stream_handle(stream)), "bl_probe_mfma_i8")


# ------------------------------------------------------------- FFN glue ---

ACT_SILU = 0        # BL_ACT_SILU: Qwen3
ACT_GELU_TANH = 1   # BL_ACT_GELU_TANH: Gemma3 (gelu_pytorch_tanh)


def bitlinear_glu_quant(gate, up, act: int, norm_w, eps: float, xq=None, x_factor=None, stream=None):
    """(int8 codes [M, K], float32 factor [M]) of the down projection's input
    act(gate) * up (formed in registers, never stored)."""
    torch = _torch()
    M, K = gate.shape
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=gate.device)
    if x_factor is None:
        x_factor = torch.empty((M,), dtype=torch.float32, device=gate.device)
    nw, f16 = _norm(norm_w, K)
    fn = _lib.bitlinear_glu_quant_nwf16 if f16 else _lib.bitlinear_glu_quant
    _check(fn(
        _dev(gate, torch.float32, "gate"), _dev(up, torch.float32, "up", (M, K)), act,
        nw, M, K, eps, _dev(xq, torch.int8, "xq", (M, K)),
        _dev(x_factor, torch.float32, "x_factor", (M,)), _stream_handle(stream)),
        "bitlinear_glu_quant")
    return xq, x_factor


def bitlinear_glu_forward(gate, up, act: int, norm_w, packed_w, w_scale: float, N: int, eps: float,
                          y=None, stream=None):
    """y[M, N] = BitLinear_down(act(gate) * up) on the GPU; returns y."""
    torch = _torch()
    M, K = gate.shape
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=gate.device)
    nw, f16 = _norm(norm_w, K)
    fn = _lib.bitlinear_glu_forward_nwf16 if f16 else _lib.bitlinear_glu_forward
    _check(fn(
        _dev(gate, torch.float32, "gate"), _dev(up, torch.float32, "up", (M, K)), act,
        nw, _dev(packed_w, torch.uint8, "packed_w"),
        w_scale, M, K, N, eps, _dev(y, torch.float32, "y", (M, N)), _stream_handle(stream)),
        "bitlinear_glu_forward")
    return y
