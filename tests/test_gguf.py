"""bl_gguf_find_tensor (host): I2_S and float16/float32 tensors located in GGUF
file images written by tests/gguf_file.py; malformed and truncated images
rejected.  The I2_S payload read back is the oracle's packed buffer itself,
so a projection can run from a model file.  Parity with real bitnet.cpp files
stays unpinned: none is available here."""
import ctypes

import numpy as np
import pytest

import gguf_file as gg
import oracle
from ternary_weight_amd import bitlinear as bl
from ternary_weight_amd import inputs


def _layer_image(alignment=32, version=3, extra_kv=()):
    K, N = 1024, 2048
    W = inputs.weight(31, 0, 0, N, K)
    packed, scale = oracle.i2s_pack(W)
    nw = inputs.norm_weight(31, 0, 0, K)
    out_norm = inputs.norm_weight(31, 0, 1, K)
    kvs = [("general.architecture", gg.STRING, "qwen3"),
           ("qwen3.block_count", gg.U32, 28),
           ("qwen3.attention.layer_norm_rms_epsilon", gg.F32, 1e-6),
           ("tokenizer.ggml.tokens", gg.ARRAY, (gg.STRING, ["<a>", "b", "cc"])),
           ("tokenizer.ggml.scores", gg.ARRAY, (gg.F32, [0.5, -1.0, 2.0])),
           ("tokenizer.ggml.add_eos_token", gg.BOOL, True),
           ("general.file_type", gg.U64, 40), ("x.i8", gg.I8, -3), ("x.f64", gg.F64, 2.5),
           *extra_kv]
    if alignment != 32:
        kvs.append(("general.alignment", gg.U32, alignment))
    tensors = [("output_norm.weight", gg.T_F32, [K], out_norm.tobytes()),
               ("blk.0.attn_q.weight", gg.T_I2S, [K, N], packed.tobytes()),
               ("blk.0.attn_q_norm_in.weight", gg.T_F16, [K], nw.astype(np.float16).tobytes()),
               ("blk.0.q8.weight", 8, [64, 2], bytes(68))]
    img = gg.write(kvs, tensors, alignment=alignment, version=version)
    return img, dict(K=K, N=N, packed=packed, scale=scale, nw=nw, out_norm=out_norm)


@pytest.mark.parametrize("alignment,version", [(32, 3), (64, 3), (32, 2), (256, 3)])
def test_find_tensors(alignment, version):
    img, ref = _layer_image(alignment, version)
    q = bl.gguf_find_tensor(img, "blk.0.attn_q.weight")
    assert q["type"] == bl.GGUF_I2S and q["dims"] == [ref["K"], ref["N"]]
    assert q["offset"] % alignment == 0
    assert q["nbytes"] == bl.i2s_packed_bytes(ref["K"], ref["N"]) == ref["packed"].size
    buf, scale, K, N = bl.gguf_i2s_weight(img, "blk.0.attn_q.weight")
    assert (K, N) == (ref["K"], ref["N"]) and scale == ref["scale"]
    assert np.array_equal(buf, ref["packed"])
    n = bl.gguf_find_tensor(img, "blk.0.attn_q_norm_in.weight")
    assert n["type"] == bl.GGUF_F16 and n["dims"] == [ref["K"]] and n["nbytes"] == 2 * ref["K"]
    half = img[n["offset"]:n["offset"] + n["nbytes"]].view(np.uint16)
    assert np.array_equal(oracle.half_to_float(half), ref["nw"].astype(np.float16).astype(np.float32))
    o = bl.gguf_find_tensor(img, "output_norm.weight")
    assert o["type"] == bl.GGUF_F32
    assert np.array_equal(img[o["offset"]:o["offset"] + o["nbytes"]].view(np.float32), ref["out_norm"])
    u = bl.gguf_find_tensor(img, "blk.0.q8.weight")
    assert u["type"] == 8 and u["nbytes"] == 0  # a type this library does not size


def test_projection_from_file_matches_oracle():
    # The oracle's forward on the weight read back from the file, with the
    # float16 norm weight from the file, equals the one on the original
    # buffers (same bytes, same widened norm).
    img, ref = _layer_image()
    buf, scale, K, N = bl.gguf_i2s_weight(img, "blk.0.attn_q.weight")
    n = bl.gguf_find_tensor(img, "blk.0.attn_q_norm_in.weight")
    nw = oracle.half_to_float(img[n["offset"]:n["offset"] + n["nbytes"]].view(np.uint16))
    x = inputs.activations(31, 0, 2, 3, K)
    y_file = oracle.bitlinear(x, nw, np.ascontiguousarray(buf), N, inputs.EPS)
    y_ref = oracle.bitlinear(x, ref["nw"].astype(np.float16).astype(np.float32), ref["packed"], N,
                             inputs.EPS)
    assert np.array_equal(y_file, y_ref)


def _status(img, name):
    t = bl.GgufTensor()
    img = np.ascontiguousarray(img, dtype=np.uint8)
    return bl.lib.bl_gguf_find_tensor(img.ctypes.data if img.size else None, img.size,
                                      name.encode(), ctypes.byref(t))


def test_errors():
    img, _ = _layer_image()
    assert _status(img, "blk.0.attn_k.weight") == bl.BL_ERR_NOT_FOUND
    bad = img.copy()
    bad[:4] = np.frombuffer(b"GGUG", np.uint8)
    assert _status(bad, "blk.0.attn_q.weight") == bl.BL_ERR_INVALID_ARGUMENT
    v1, _ = _layer_image(version=1)
    assert _status(v1, "blk.0.attn_q.weight") == bl.BL_ERR_UNSUPPORTED
    t = bl.GgufTensor()
    assert bl.lib.bl_gguf_find_tensor(None, 10, b"x", ctypes.byref(t)) == bl.BL_ERR_INVALID_ARGUMENT
    assert bl.lib.bl_gguf_find_tensor(img.ctypes.data, img.size, None, ctypes.byref(t)) == bl.BL_ERR_INVALID_ARGUMENT
    assert bl.lib.bl_gguf_find_tensor(img.ctypes.data, img.size, b"x", None) == bl.BL_ERR_INVALID_ARGUMENT
    # an unknown metadata value type
    k = gg.write([("a", gg.U32, 1)], [("w", gg.T_F32, [4], bytes(16))])
    pos = bytes(k).index(b"a") + 1  # the value type follows the key
    k2 = k.copy()
    k2[pos:pos + 4] = np.frombuffer(np.uint32(99).tobytes(), np.uint8)
    assert _status(k, "w") == bl.BL_OK
    assert _status(k2, "w") == bl.BL_ERR_INVALID_ARGUMENT
    # I2_S weights must be 2-D with whole 128-value blocks
    odd = gg.write([], [("w", gg.T_I2S, [96, 4], bytes(96 + 4))])
    assert _status(odd, "w") == bl.BL_ERR_UNSUPPORTED
    three = gg.write([], [("w", gg.T_I2S, [128, 2, 2], bytes(128 + 4))])
    assert _status(three, "w") == bl.BL_ERR_UNSUPPORTED
    # dimension counts and zero dimensions
    z = gg.write([], [("w", gg.T_F32, [0, 4], b"")])
    assert _status(z, "w") == bl.BL_ERR_INVALID_ARGUMENT
    five = gg.write([], [("w", gg.T_F32, [1, 1, 1, 1, 1], bytes(4))])
    assert _status(five, "w") == bl.BL_ERR_INVALID_ARGUMENT
    # data running past the end of the file
    short = gg.write([], [("w", gg.T_F32, [64], bytes(256))])
    assert _status(short[:-4], "w") == bl.BL_ERR_INVALID_ARGUMENT


def test_every_truncation_is_rejected():
    # Every prefix of a small file is rejected cleanly: an error status, never
    # a read past the given size (the reader checks every access).
    img = gg.write([("general.architecture", gg.STRING, "gemma3"),
                    ("t", gg.ARRAY, (gg.STRING, ["x", "yy"])),
                    ("s", gg.ARRAY, (gg.U16, [1, 2, 3]))],
                   [("a", gg.T_F16, [128], bytes(256)),
                    ("blk.0.ffn_down.weight", gg.T_I2S, [128, 3], bytes(96 + 4))])
    assert _status(img, "blk.0.ffn_down.weight") == bl.BL_OK
    for cut in range(img.size):
        st = _status(img[:cut], "blk.0.ffn_down.weight")
        assert st in (bl.BL_ERR_INVALID_ARGUMENT,), (cut, st)
