"""Plain CPU oracle for the BitLinear forward path with I2_S ternary weights.

TEST INFRASTRUCTURE ONLY: this package may be imported only by ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``.  The
product path (``ternary_weight_amd``) never imports it, and it never imports
the product path.  The arithmetic lives in ``bitlinear_oracle.c`` (plain C,
single-threaded, double precision where the pages leave precision open); this
module only builds it with gcc and marshals numpy arrays.

Pages followed (by title and section):
  * "BitNet Embeddings GGUF Conversion Implementation", s1 "Background",
    s3 "I2_S Ternary Packing", s4.5 "load_tensors".
  * "BitNet Inference Framework", "Quantization and Encoding", "Data Layout",
    "Quantization (W1.58A8)", "Architectural Details".
  * "gguf-gemv", "Requirements".
  * "BitNet Embeddings GGUF Conversion Implementation", s4.5 FFN per-projection
    norms (act(gate) * up feeding the down projection) and the s1 model table
    (SiLU for Qwen3, gelu_pytorch_tanh for Gemma3).
  * "BitNet Embeddings GGUF Conversion Implementation", s3 tensor type table
    and s6.1 "F16 Norm Weight Support" (norm weights stored as float16).

Every function is pinned by ``tests/test_oracle_pins.py`` to values fixed by
the pages' definitions and by mathematics (hand-worked examples, closed forms,
invariants and brute force), not to itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitlinear_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

REF_OK = 0
REF_ERR_ARG = -1
REF_ERR_CODE3 = -2
REF_ERR_OVERFLOW = -3
REF_ERR_NOMEM = -4
REF_ERR_NONFINITE = -5

ACT_SILU = 0        # Qwen3
ACT_GELU_TANH = 1   # Gemma3 (gelu_pytorch_tanh)


def build() -> str:
    """Compile the oracle with gcc: -O2, no fast-math, no FMA contraction."""
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.ref_i2s_packed_bytes.argtypes = [i64, i64]
        lib.ref_i2s_packed_bytes.restype = i64
        lib.ref_i2s_pack.argtypes = [p, i64, i64, p, p]
        lib.ref_i2s_unpack.argtypes = [p, i64, i64, p, p]
        lib.ref_quant.argtypes = [p, p, i64, i64, ctypes.c_float, p, p]
        lib.ref_matmul_i32.argtypes = [p, p, i64, i64, i64, p]
        lib.ref_epilogue.argtypes = [p, p, ctypes.c_float, i64, i64, p]
        lib.ref_epilogue.restype = None
        lib.ref_bitlinear.argtypes = [p, p, p, i64, i64, i64, ctypes.c_float, p]
        lib.ref_act.argtypes = [ctypes.c_int, ctypes.c_double]
        lib.ref_act.restype = ctypes.c_double
        lib.ref_glu.argtypes = [p, p, ctypes.c_int, i64, p]
        lib.ref_glu_quant.argtypes = [p, p, ctypes.c_int, p, i64, i64, ctypes.c_float, p, p]
        lib.ref_glu_bitlinear.argtypes = [p, p, ctypes.c_int, p, p, i64, i64, i64, ctypes.c_float, p]
        lib.ref_half_to_float.argtypes = [p, i64, p]
        lib.ref_half_to_float.restype = None
        for name in ("ref_i2s_pack", "ref_i2s_unpack", "ref_quant", "ref_matmul_i32",
                     "ref_bitlinear", "ref_glu", "ref_glu_quant", "ref_glu_bitlinear"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


class OracleError(RuntimeError):
    pass


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != REF_OK:
        raise OracleError(f"{what} failed with code {rc}")


def packed_bytes(K: int, N: int) -> int:
    return int(_load().ref_i2s_packed_bytes(K, N))


def i2s_pack(w: np.ndarray) -> tuple[np.ndarray, float]:
    """W float32 [N, K] -> (packed uint8 [N*K/4 + 4], scale float)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    nbytes = packed_bytes(K, N)
    if nbytes == 0:
        raise OracleError(f"invalid shape N={N} K={K}")
    out = np.zeros(nbytes, dtype=np.uint8)
    scale = np.zeros(1, dtype=np.float32)
    _check(_load().ref_i2s_pack(_ptr(w), K, N, _ptr(out), _ptr(scale)), "ref_i2s_pack")
    return out, float(scale[0])


def i2s_unpack(packed: np.ndarray, K: int, N: int) -> tuple[np.ndarray, float]:
    """Packed bytes -> (ternary int8 [N, K] in {-1,0,1}, stored scale)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    q = np.zeros((N, K), dtype=np.int8)
    scale = np.zeros(1, dtype=np.float32)
    _check(_load().ref_i2s_unpack(_ptr(packed), K, N, _ptr(q), _ptr(scale)), "ref_i2s_unpack")
    return q, float(scale[0])


def half_to_float(h: np.ndarray) -> np.ndarray:
    """IEEE binary16 values (a float16 array, or their uint16 bit patterns)
    widened to float32 by the oracle's own decoder."""
    bits = np.ascontiguousarray(np.asarray(h).view(np.uint16) if np.asarray(h).dtype == np.float16
                                else np.asarray(h, dtype=np.uint16))
    out = np.empty(bits.shape, dtype=np.float32)
    _load().ref_half_to_float(_ptr(bits), bits.size, _ptr(out))
    return out


def _norm(norm_w):
    """norm_w as float32 (None: no per-projection norm) and its pointer.  A
    float16 norm weight is widened exactly first (its stored dtype in the
    pages' GGUF files)."""
    if norm_w is None:
        return None, None
    if np.asarray(norm_w).dtype == np.float16:
        norm_w = half_to_float(norm_w)
    norm_w = np.ascontiguousarray(norm_w, dtype=np.float32)
    return norm_w, _ptr(norm_w)


def quant(x: np.ndarray, norm_w, eps: float) -> tuple[np.ndarray, np.ndarray]:
    """x float32 [M, K], norm_w float32 [K] or None -> (int8 codes [M, K], float64 factor [M])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    norm_w, pn = _norm(norm_w)
    M, K = x.shape
    q = np.zeros((M, K), dtype=np.int8)
    factor = np.zeros(M, dtype=np.float64)
    _check(_load().ref_quant(_ptr(x), pn, M, K, eps, _ptr(q), _ptr(factor)), "ref_quant")
    return q, factor


def matmul_i32(xq: np.ndarray, packed: np.ndarray, K: int, N: int) -> np.ndarray:
    """int8 codes [M, K] x packed weights -> int32 [M, N]."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    M = xq.shape[0]
    acc = np.zeros((M, N), dtype=np.int32)
    _check(_load().ref_matmul_i32(_ptr(xq), _ptr(packed), M, K, N, _ptr(acc)), "ref_matmul_i32")
    return acc


def epilogue(acc: np.ndarray, factor: np.ndarray, scale: float) -> np.ndarray:
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    factor = np.ascontiguousarray(factor, dtype=np.float64)
    M, N = acc.shape
    y = np.zeros((M, N), dtype=np.float32)
    _load().ref_epilogue(_ptr(acc), _ptr(factor), scale, M, N, _ptr(y))
    return y


def bitlinear(x: np.ndarray, norm_w, packed: np.ndarray, N: int,
              eps: float) -> np.ndarray:
    """The whole forward path: float32 [M, K] -> float32 [M, N] (norm_w None: no norm)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    norm_w, pn = _norm(norm_w)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    M, K = x.shape
    y = np.zeros((M, N), dtype=np.float32)
    _check(_load().ref_bitlinear(_ptr(x), pn, _ptr(packed), M, K, N, eps, _ptr(y)),
           "ref_bitlinear")
    return y


def act(kind: int, z: float) -> float:
    """The FFN activation at one point, in double (ACT_SILU or ACT_GELU_TANH)."""
    return float(_load().ref_act(kind, z))


def glu(gate: np.ndarray, up: np.ndarray, kind: int) -> np.ndarray:
    """act(gate) * up elementwise, float64 (same shape as gate)."""
    gate = np.ascontiguousarray(gate, dtype=np.float32)
    up = np.ascontiguousarray(up, dtype=np.float32)
    assert gate.shape == up.shape
    h = np.zeros(gate.shape, dtype=np.float64)
    _check(_load().ref_glu(_ptr(gate), _ptr(up), kind, gate.size, _ptr(h)), "ref_glu")
    return h


def glu_quant(gate: np.ndarray, up: np.ndarray, kind: int, norm_w: np.ndarray,
              eps: float) -> tuple[np.ndarray, np.ndarray]:
    """Down-projection input steps on act(gate) * up: (int8 codes [M, K], float64 factor [M])."""
    gate = np.ascontiguousarray(gate, dtype=np.float32)
    up = np.ascontiguousarray(up, dtype=np.float32)
    norm_w, pn = _norm(norm_w)
    M, K = gate.shape
    q = np.zeros((M, K), dtype=np.int8)
    factor = np.zeros(M, dtype=np.float64)
    _check(_load().ref_glu_quant(_ptr(gate), _ptr(up), kind, pn, M, K, eps, _ptr(q),
                                 _ptr(factor)), "ref_glu_quant")
    return q, factor


def glu_bitlinear(gate: np.ndarray, up: np.ndarray, kind: int, norm_w: np.ndarray,
                  packed: np.ndarray, N: int, eps: float) -> np.ndarray:
    """The down projection fed by act(gate) * up: float32 [M, K] pair -> float32 [M, N]."""
    gate = np.ascontiguousarray(gate, dtype=np.float32)
    up = np.ascontiguousarray(up, dtype=np.float32)
    norm_w, pn = _norm(norm_w)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    M, K = gate.shape
    y = np.zeros((M, N), dtype=np.float32)
    _check(_load().ref_glu_bitlinear(_ptr(gate), _ptr(up), kind, pn, _ptr(packed), M, K,
                                     N, eps, _ptr(y)), "ref_glu_bitlinear")
    return y
