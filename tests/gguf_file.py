"""A minimal GGUF writer for the tests (little-endian, versions 2 and 3):
metadata key/value pairs of any scalar, string or array type, then tensor
infos, then the data section aligned to `alignment` with each tensor's data
at an aligned offset.  Written from the container's published layout, apart
from the library's reader; only tests use it.

I2_S tensors (type 36) are written as their packed buffer as it stands: the
code bytes followed by the float32 scale ("BitNet Embeddings GGUF Conversion
Implementation", s3 "I2_S Ternary Packing" and s6.2 "gguf-py: I2_S Type").
"""
from __future__ import annotations

import struct

import numpy as np

U8, I8, U16, I16, U32, I32, F32, BOOL, STRING, ARRAY, U64, I64, F64 = range(13)
_FMT = {U8: "<B", I8: "<b", U16: "<H", I16: "<h", U32: "<I", I32: "<i", F32: "<f", BOOL: "<?",
        U64: "<Q", I64: "<q", F64: "<d"}
T_F32, T_F16, T_I2S = 0, 1, 36


def _str(s: str) -> bytes:
    b = s.encode()
    return struct.pack("<Q", len(b)) + b


def _value(vtype: int, v) -> bytes:
    if vtype == STRING:
        return _str(v)
    if vtype == ARRAY:
        etype, items = v
        out = struct.pack("<IQ", etype, len(items))
        return out + b"".join(_value(etype, x) for x in items)
    return struct.pack(_FMT[vtype], v)


def write(kvs, tensors, alignment: int = 32, version: int = 3, magic: bytes = b"GGUF") -> np.ndarray:
    """kvs: [(key, vtype, value)]; tensors: [(name, type, dims innermost
    first, data bytes)].  Returns the file image as a uint8 array."""
    head = magic + struct.pack("<IQQ", version, len(tensors), len(kvs))
    for key, vtype, value in kvs:
        head += _str(key) + struct.pack("<I", vtype) + _value(vtype, value)
    offsets, off = [], 0
    for _, _, _, data in tensors:
        off = (off + alignment - 1) // alignment * alignment
        offsets.append(off)
        off += len(data)
    for (name, ttype, dims, _), o in zip(tensors, offsets):
        head += _str(name) + struct.pack("<I", len(dims)) + struct.pack(f"<{len(dims)}Q", *dims)
        head += struct.pack("<IQ", ttype, o)
    start = (len(head) + alignment - 1) // alignment * alignment
    img = bytearray(head) + bytearray(start - len(head))
    for (_, _, _, data), o in zip(tensors, offsets):
        img += bytearray(start + o - len(img))
        img += bytes(data)
    return np.frombuffer(bytes(img), dtype=np.uint8).copy()
