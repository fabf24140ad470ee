"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Criteria (the path's stated tolerances):
  * integer product: bit-exact when both sides get the same int8 codes;
  * fused quantization: codes differ by at most 1, on at most 0.01% of the
    elements of a case, and only where the double-precision value lies within
    1e-4 of a rounding boundary; factor relative error <= 1e-6;
  * output: relative L2 error <= 1e-3 per projection.
Large workloads are checked on sampled rows (rows are independent: the
quantization is per token), always including the first and the last row.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from ternary_weight_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bl = pytest.importorskip("ternary_weight_amd.bitlinear")

DEV = "cuda"
EPS = inputs.EPS


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def rel_l2(a, b) -> float:
    a = a.astype(np.float64)
    b = b.astype(np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def check_codes(q_gpu, q_ref, x, norm_w):
    """|dq| <= 1, flips <= 0.01% of elements, each flip next to a rounding tie."""
    d = q_gpu.astype(np.int32) - q_ref.astype(np.int32)
    assert np.abs(d).max(initial=0) <= 1
    flips = np.argwhere(d != 0)
    assert len(flips) <= 1e-4 * d.size, f"{len(flips)} code flips in {d.size}"
    for m, k in flips:
        u = x[m].astype(np.float64) * norm_w.astype(np.float64)
        v = u[k] * 127.0 / np.abs(u).max()
        assert abs(abs(v - math.floor(v)) - 0.5) < 1e-4, f"flip away from a tie at ({m},{k}): {v}"
    return len(flips)


def check_factor(f_gpu, f_ref):
    f_ref = np.asarray(f_ref, np.float64)
    err = np.abs(f_gpu.astype(np.float64) - f_ref)
    assert np.all(err <= 1e-6 * np.abs(f_ref)), float((err / np.maximum(f_ref, 1e-300)).max())


def proj_inputs(wl, layer, pi, M, K, N, heavy=False):
    W = inputs.weight(wl, layer, pi, N, K)
    packed, scale = oracle.i2s_pack(W)
    nw = inputs.norm_weight(wl, layer, pi, K)
    x = inputs.activations(wl, layer, pi, M, K, heavy)
    return x, nw, packed, scale


# ------------------------------------------------------------ quantization ---

QUANT_CASES = [(1, 1024), (8, 1024), (5, 128), (512, 640), (512, 1024), (257, 2048),
               (300, 3072), (7, 4096), (3, 8192), (2, 16384)]


@pytest.mark.parametrize("M,K", QUANT_CASES)
def test_quant_parity(M, K):
    x = inputs.activations(11, 0, K, M, K)
    nw = inputs.norm_weight(11, 0, K, K)
    xq, f = bl.bitlinear_quant(dev(x), dev(nw), EPS)
    q_ref, f_ref = oracle.quant(x, nw, EPS)
    flips = check_codes(host(xq), q_ref, x, nw)
    check_factor(host(f), f_ref)
    log(f"quant M={M} K={K}: {flips} flips")


def test_quant_heavy_tail_and_special_rows():
    M, K = 1024, 3072
    x = inputs.activations(5, 0, 6, M, K, heavy_tail=True)
    x[3] = 0.0                 # all-zero row
    x[4] = 1e-35               # tiny row: 127/absmax overflows float32
    x[5, :] = 0.0
    x[5, 17] = -2.5            # one non-zero element
    nw = inputs.norm_weight(5, 0, 6, K)
    xq, f = bl.bitlinear_quant(dev(x), dev(nw), EPS)
    q_ref, f_ref = oracle.quant(x, nw, EPS)
    q = host(xq)
    assert np.all(q[3] == 0) and host(f)[3] == 0.0
    assert q[5, 17] == -127 and np.count_nonzero(q[5]) == 1
    check_codes(q, q_ref, x, nw)
    check_factor(host(f), f_ref)


# ---------------------------------------------------------- integer product ---

MATMUL_CASES = [
    # decode kernel (M <= 16)
    (1, 1024, 3072), (2, 128, 1), (3, 640, 5), (4, 1024, 1024), (5, 3072, 1024), (6, 2048, 1024),
    (7, 384, 67), (8, 1024, 3072), (9, 256, 130), (15, 1152, 64), (16, 4096, 48),
    # tiled MFMA kernel
    (17, 128, 1), (17, 1024, 1024), (64, 640, 256), (200, 1280, 333), (255, 2048, 640),
    (257, 640, 2048), (512, 3072, 1024), (130, 8192, 129),
    # the Gemma3-270M layer at M = 512 (q, k/v, o, gate/up, down)
    (512, 640, 1024), (512, 640, 256), (512, 1024, 640), (512, 640, 2048), (512, 2048, 640),
    # decode rows too long to stage in LDS: activation fragments from global
    # memory (M*K > 64 KB), with even and odd superblock counts
    (16, 8192, 96), (9, 8064, 130), (12, 65536, 8), (9, 4224, 130),
]


@pytest.mark.parametrize("M,K,N", MATMUL_CASES)
def test_matmul_i32_bit_exact(M, K, N):
    W = inputs.weight(12, M, K, N, K)
    packed, _ = oracle.i2s_pack(W)
    xq = inputs.rng(12, M, K, 7).integers(-127, 128, size=(M, K)).astype(np.int8)
    acc = bl.bitlinear_matmul_i32(dev(xq), dev(packed), N)
    ref = oracle.matmul_i32(xq, packed, K, N)
    assert np.array_equal(host(acc), ref)


@pytest.mark.parametrize("M", [1, 16, 17, 300])
def test_matmul_i32_extremes(M):
    K, N = 2048, 96
    ones, _ = oracle.i2s_pack(np.ones((N, K), np.float32))
    xq = np.full((M, K), 127, np.int8)
    xq[1::2] = -127
    acc = host(bl.bitlinear_matmul_i32(dev(xq), dev(ones), N))
    assert np.array_equal(acc, oracle.matmul_i32(xq, ones, K, N))
    assert acc[0, 0] == 127 * K and (M < 2 or acc[1, 0] == -127 * K)
    zero, _ = oracle.i2s_pack(np.zeros((N, K), np.float32))
    assert np.all(host(bl.bitlinear_matmul_i32(dev(xq), dev(zero), N)) == 0)


@pytest.mark.parametrize("M,K,N", [(1, 128, 40000), (2, 128, 100000), (3, 256, 33000), (16, 1024, 36000)])
def test_decode_single_call_wide_n(M, K, N):
    # A single-problem decode launch gives each workgroup as few 64-row tiles
    # as keep about 512 workgroups busy: one below N = 32768, 2..4 here.  The
    # same problems in a group take the full tile count per workgroup; the
    # results agree bit for bit, and with the oracle.
    x, nw, packed, scale = proj_inputs(16, M, K, M, K, N)
    dx, dn, dp = dev(x), dev(nw), dev(packed)
    xq, _ = bl.bitlinear_quant(dx, dn, EPS)
    acc = bl.bitlinear_matmul_i32(xq, dp, N)
    assert np.array_equal(host(acc), oracle.matmul_i32(host(xq), packed, K, N))
    y = bl.bitlinear_forward(dx, dn, dp, scale, N, EPS)
    assert rel_l2(host(y), oracle.bitlinear(x, nw, packed, N, EPS)) <= 1e-3
    it = dict(x=dx, norm_w=dn, packed_w=dp, w_scale=scale, eps=EPS, N=N,
              y=torch.full((M, N), float("nan"), device=DEV))
    with bl.Group([it]) as g:
        g.forward()
        torch.cuda.synchronize()
        assert torch.equal(it["y"], y)


@pytest.mark.parametrize("M,K,N", [(16, 8192, 200), (11, 8064, 77)])
def test_decode_long_rows_from_global(M, K, N):
    # Decode rows longer than the 64 KB activation staging: the fragments are
    # read from global memory.  Single call and a group table (the other
    # kernel instance) against the oracle and the hooks, bit for bit.
    x, nw, packed, scale = proj_inputs(23, M, K, M, K, N)
    x[M // 2] = 0.0
    dx, dn, dp = dev(x), dev(nw), dev(packed)
    y = bl.bitlinear_forward(dx, dn, dp, scale, N, EPS)
    xq, f = bl.bitlinear_quant(dx, dn, EPS)
    acc = bl.bitlinear_matmul_i32(xq, dp, N)
    assert np.array_equal(host(acc), oracle.matmul_i32(host(xq), packed, K, N))
    assert torch.equal(y, _hooks_epilogue(acc, f, scale))
    assert rel_l2(host(y), oracle.bitlinear(x, nw, packed, N, EPS)) <= 1e-3
    it = dict(x=dx, norm_w=dn, packed_w=dp, w_scale=scale, eps=EPS, N=N,
              y=torch.full((M, N), float("nan"), device=DEV))
    other = dict(x=dev(x[:1].copy()), norm_w=dn, packed_w=dp, w_scale=scale, eps=EPS, N=N,
                 y=torch.full((1, N), float("nan"), device=DEV))
    with bl.Group([it, other]) as g:
        assert [d["kind"] for d in g.forward_launches()] == ["quant", "decode"]
        g.forward()
        torch.cuda.synchronize()
        assert torch.equal(it["y"], y)
        assert torch.equal(other["y"], bl.bitlinear_forward(other["x"], dn, dp, scale, N, EPS))


def _valid_i2s_bytes(rng, n: int) -> np.ndarray:
    """n random packed bytes whose four 2-bit fields are codes 0, 1 or 2."""
    valid = np.array([(a << 6) | (b << 4) | (c << 2) | d for a in range(3) for b in range(3)
                      for c in range(3) for d in range(3)], dtype=np.uint8)
    return valid[rng.integers(0, valid.size, size=n, dtype=np.uint8)]


def _rows_with_tail(packed: np.ndarray, K: int, n0: int, n1: int) -> np.ndarray:
    """Weight rows n0..n1-1 of a packed buffer, with its scale tail appended."""
    rb = K // 4
    return np.concatenate([packed[n0 * rb:n1 * rb], packed[-4:]])


# The widest weight the library accepts: N*K/4 packed bytes exactly at the
# 32-bit offset limit (2^31 - 4096), for the decode and the prefill kernel.
N_AT_OFFSET_LIMIT = ((1 << 31) - 4096) // 32


@pytest.mark.parametrize("M,K,N", [(20, 128, (1 << 22) + 300), (40, 65536, 70),
                                   (1, 128, N_AT_OFFSET_LIMIT), (20, 128, N_AT_OFFSET_LIMIT)])
def test_extreme_shapes(M, K, N):
    # Paths that the workloads never reach: an output wider than the
    # prefill kernel's full-tile store path allows (more than 2^22 columns:
    # every tile takes the bounds-checked stores, the last one ragged), the
    # longest K the library accepts (512 K blocks per tile; its quantization
    # streams the row), and the widest weight it accepts (N*K/4 bytes at the
    # 32-bit offset limit) through the decode and the prefill kernel.  Raw
    # int32 products against the oracle on column ranges at both ends and
    # around 2^22, the forward bit-identical to the hooks' composition
    # everywhere and within 1e-3 of the oracle on those ranges.
    rng = inputs.rng(31, M, K, 1)
    rb = K // 4
    packed = np.concatenate([_valid_i2s_bytes(rng, N * rb),
                             np.frombuffer(np.float32(41.5).tobytes(), np.uint8)])
    scale = 41.5
    xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    x = inputs.activations(31, 0, M, M, K)
    nw = inputs.norm_weight(31, 0, M, K)
    dp = dev(packed)
    ranges = [(0, min(N, 256)), (max(0, N - 300), N)]
    if N > (1 << 22):
        ranges.append(((1 << 22) - 128, (1 << 22) + 256))
    acc = bl.bitlinear_matmul_i32(dev(xq), dp, N)
    for n0, n1 in ranges:
        ref = oracle.matmul_i32(xq, _rows_with_tail(packed, K, n0, n1), K, n1 - n0)
        assert np.array_equal(host(acc[:, n0:n1]), ref), f"int32 columns {n0}..{n1}"
    del acc
    dx, dn = dev(x), dev(nw)
    y = bl.bitlinear_forward(dx, dn, dp, scale, N, EPS)
    q, f = bl.bitlinear_quant(dx, dn, EPS)
    acc = bl.bitlinear_matmul_i32(q, dp, N)
    assert torch.equal(y, _hooks_epilogue(acc, f, scale))
    del acc
    for n0, n1 in ranges:
        y_ref = oracle.bitlinear(x, nw, _rows_with_tail(packed, K, n0, n1), n1 - n0, EPS)
        assert rel_l2(host(y[:, n0:n1]), y_ref) <= 1e-3, f"forward columns {n0}..{n1}"


def test_activation_offset_limit():
    # The most activation codes the library accepts: M*K just below the
    # 32-bit offset limit (M = 32767 rows of K = 65536: 2.1 G codes from 8.6 GB
    # of fp32 rows), through the streaming quantization and the prefill
    # kernel, into a NaN-filled output.  The forward equals the fp32 epilogue
    # of the hooks everywhere; one row in every 128-row tile is checked
    # against the oracle (codes and factor, the int32 product of the GPU's
    # codes bit-exactly, the forward within 1e-3).
    K, N = 65536, 8
    M = ((1 << 31) - 4096) // K
    x = inputs.activations_device(torch, 32, 0, 0, M, K, DEV)
    nw = inputs.norm_weight(32, 0, 0, K)
    packed, scale = oracle.i2s_pack(inputs.weight(32, 0, 0, N, K))
    dn, dp = dev(nw), dev(packed)
    y = torch.full((M, N), float("nan"), device=DEV)
    bl.bitlinear_forward(x, dn, dp, scale, N, EPS, y=y)
    assert bool(torch.isfinite(y).all())
    xq, f = bl.bitlinear_quant(x, dn, EPS)
    acc = bl.bitlinear_matmul_i32(xq, dp, N)
    assert torch.equal(y, _hooks_epilogue(acc, f, scale))
    rows = inputs.tile_rows(M, 128, seed=32)
    idx = torch.as_tensor(rows, device=DEV)
    xr = host(x[idx])
    q_gpu = host(xq[idx])
    q_ref, f_ref = oracle.quant(xr, nw, EPS)
    check_codes(q_gpu, q_ref, xr, nw)
    check_factor(host(f[idx]), f_ref)
    assert np.array_equal(host(acc[idx]), oracle.matmul_i32(q_gpu, packed, K, N))
    assert rel_l2(host(y[idx]), oracle.bitlinear(xr, nw, packed, N, EPS)) <= 1e-3


def _hooks_epilogue(acc, f, scale):
    """The forward's fp32 epilogue applied to the hooks' results: float(acc)
    times (factor / w_scale), each step one fp32 rounding."""
    return acc.to(torch.float32) * (f / torch.tensor(scale, dtype=torch.float32, device=DEV))[:, None]


# ------------------------------------------------------------ whole path ---

def forward_and_check(x, nw, packed, scale, N, tag):
    y = bl.bitlinear_forward(dev(x), dev(nw), dev(packed), scale, N, EPS)
    y_ref = oracle.bitlinear(x, nw, packed, N, EPS)
    err = rel_l2(host(y), y_ref)
    assert err <= 1e-3, f"{tag}: rel L2 {err}"
    return err


@pytest.mark.parametrize("wid", [1, 2, 3])
def test_forward_small_workloads_full(wid):
    w = inputs.WORKLOADS[wid]
    for pi, (name, K, N) in enumerate(w.projs):
        x, nw, packed, scale = proj_inputs(wid, 0, pi, w.M, K, N)
        err = forward_and_check(x, nw, packed, scale, N, f"w{wid} {name}")
        log(f"workload {wid} {name} M={w.M} K={K} N={N}: rel L2 {err:.2e}")


EDGE_M = [1, 2, 3, 4, 5, 6, 7, 8, 9, 15, 16, 17, 255, 257]


@pytest.mark.parametrize("M", EDGE_M)
def test_forward_edge_rows(M):
    K, N = 384, 37  # ragged N, three I2_S blocks
    x, nw, packed, scale = proj_inputs(13, M, 0, M, K, N)
    x[M // 2] = 0.0  # a zero row inside the batch
    y = host(bl.bitlinear_forward(dev(x), dev(nw), dev(packed), scale, N, EPS))
    y_ref = oracle.bitlinear(x, nw, packed, N, EPS)
    assert np.all(y[M // 2] == 0.0)
    assert rel_l2(y, y_ref) <= 1e-3


@pytest.mark.parametrize("M,K,N", [(1, 128, 1), (20, 128, 1), (3, 128, 4), (33, 640, 8)])
def test_forward_tiny_and_zero_weight(M, K, N):
    x, nw, packed, scale = proj_inputs(14, M, K, M, K, N)
    y = host(bl.bitlinear_forward(dev(x), dev(nw), dev(packed), scale, N, EPS))
    assert rel_l2(y, oracle.bitlinear(x, nw, packed, N, EPS)) <= 1e-3
    zp, zs = oracle.i2s_pack(np.zeros((N, K), np.float32))
    assert np.all(host(bl.bitlinear_forward(dev(x), dev(nw), dev(zp), zs, N, EPS)) == 0.0)


def test_hooks_compose_to_forward_bitwise():
    # forward == fp32 epilogue of (matmul_i32 o quant): same kernels, same
    # rounding steps (acc -> float, times factor/w_scale).
    for M in (4, 100):
        K, N = 1024, 256
        x, nw, packed, scale = proj_inputs(15, M, 0, M, K, N)
        dx, dn, dp = dev(x), dev(nw), dev(packed)
        y = bl.bitlinear_forward(dx, dn, dp, scale, N, EPS)
        xq, f = bl.bitlinear_quant(dx, dn, EPS)
        acc = bl.bitlinear_matmul_i32(xq, dp, N)
        y2 = acc.to(torch.float32) * (f / torch.tensor(scale, dtype=torch.float32, device=DEV))[:, None]
        assert torch.equal(y, y2)


COMPOSE_CASES = [(M, K) for K in (640, 1152, 3072, 4096) for M in (1, 2, 3, 4, 5, 8, 9, 13, 16)]


@pytest.mark.parametrize("M,K", COMPOSE_CASES)
def test_forward_matches_hooks_bitwise(M, K):
    # forward == fp32 epilogue of matmul_i32 o quant over decode shapes with
    # half superblocks; rows: heavy tailed, one all-zero, one tiny (the
    # double-precision code path), one one-hot.
    N = 96
    x, nw, packed, scale = proj_inputs(17, M, K, M, K, N, heavy=True)
    x[M // 2] = 0.0
    if M > 2:
        x[1] *= 1e-36
    if M > 3:
        x[3] = 0.0
        x[3, K // 3] = -2.5
    dx, dn, dp = dev(x), dev(nw), dev(packed)
    y = bl.bitlinear_forward(dx, dn, dp, scale, N, EPS)
    xq, f = bl.bitlinear_quant(dx, dn, EPS)
    acc = bl.bitlinear_matmul_i32(xq, dp, N)
    y2 = acc.to(torch.float32) * (f / torch.tensor(scale, dtype=torch.float32, device=DEV))[:, None]
    assert torch.equal(y, y2)
    assert rel_l2(host(y), oracle.bitlinear(x, nw, packed, N, EPS)) <= 1e-3
    # A group fuses every decode problem whose rows fit on chip (single calls
    # only up to M = 3): its in-kernel quantization must give the same bits.
    it = dict(x=dx, norm_w=dn, packed_w=dp, w_scale=scale, eps=EPS, N=N,
              y=torch.full((M, N), float("nan"), device=DEV))
    with bl.Group([it]) as g:
        g.forward()
        torch.cuda.synchronize()
        assert torch.equal(it["y"], y2)


# bitlinear_forward_prefill_fused: the quantization inside the prefill
# product's producer (a statistics pass, then the tiled kernel codes the fp32
# rows itself).  Bit-identical to bitlinear_forward (pinned to the oracle
# above) on full and ragged tiles, K up to 4096, every norm-weight kind, an
# all-zero row and a tiny row (the double-precision code path); decode sizes
# run bitlinear_forward's own path.
PQ_CASES = [(8, 1024, 3072), (17, 128, 1), (40, 1024, 72), (200, 1280, 333), (255, 2048, 640),
            (257, 640, 2048), (512, 3072, 1024), (130, 4096, 129), (1024, 1024, 3072)]


@pytest.mark.parametrize("norm", ["f32", "f16", "none"])
@pytest.mark.parametrize("M,K,N", PQ_CASES)
def test_prefill_fused_matches_forward(M, K, N, norm):
    x, nw, packed, scale = proj_inputs(19, M, K, M, K, N, heavy=True)
    x[M // 2] = 0.0
    x[1] *= 1e-36
    dx, dp = dev(x), dev(packed)
    dn = {"f32": dev(nw), "f16": torch.from_numpy(nw.astype(np.float16)).to(DEV), "none": None}[norm]
    y = bl.bitlinear_forward(dx, dn, dp, scale, N, EPS)
    y2 = torch.full((M, N), float("nan"), device=DEV)
    bl.bitlinear_forward_prefill_fused(dx, dn, dp, scale, N, EPS, y=y2)
    assert torch.equal(y, y2)
    if norm == "f32":
        assert rel_l2(host(y2), oracle.bitlinear(x, nw, packed, N, EPS)) <= 1e-3


def test_prefill_fused_full_size():
    # One Qwen3-0.6B down projection at the stack's M = 16384 (K = 3072).
    M, K, N = 16384, 3072, 1024
    x, nw, packed, scale = proj_inputs(4, 0, 6, M, K, N)
    dx, dn, dp = dev(x), dev(nw), dev(packed)
    y = bl.bitlinear_forward(dx, dn, dp, scale, N, EPS)
    y2 = torch.full((M, N), float("nan"), device=DEV)
    bl.bitlinear_forward_prefill_fused(dx, dn, dp, scale, N, EPS, y=y2)
    assert torch.equal(y, y2)


def test_group_forward_launch_kinds_and_order():
    # The forward as launches: quantization of the problems not fused (K 1024
    # -> 4 chunks, 4096 -> 16: two classes, so one merged launch for this
    # small group, bucket 0), the merged fused decode launch (3 and 4
    # superblocks: their fp32 rows fit the on-chip staging; bucket reported
    # as 0), the unfused decode launch (16 superblocks), then the prefill
    # launch.
    specs = [(1, 1024, 64), (8, 640, 40), (16, 4096, 32), (3, 1024, 48), (40, 1024, 72),
             (2, 4096, 24)]
    items, singles = [], []
    for i, (M, K, N) in enumerate(specs):
        x, nw, packed, scale = proj_inputs(18, i, 0, M, K, N)
        it = dict(x=dev(x), norm_w=dev(nw), packed_w=dev(packed), w_scale=scale, eps=EPS, N=N,
                  y=torch.full((M, N), float("nan"), device=DEV))
        items.append(it)
        singles.append(bl.bitlinear_forward(it["x"], it["norm_w"], it["packed_w"], scale, N, EPS))
    with bl.Group(items) as g:
        info = g.forward_launches()
        assert [d["kind"] for d in info] == ["quant_merged", "decode_fused", "decode", "prefill"]
        assert [d["bucket"] for d in info] == [0, 0, 16, 0]
        assert [d["count"] for d in info] == [3, 3, 2, 1]
        for i in range(len(info)):
            g.forward_launch(i)
        torch.cuda.synchronize()
        for it, ys in zip(items, singles):
            assert torch.equal(it["y"], ys)


def test_large_mixed_group():
    # About 2000 64-row blocks over 40 decode problems of mixed K (1 to 16
    # superblocks, half superblocks), M and ragged N, in one group: the same
    # results as separate calls and, on sampled problems, the oracle's.
    Ks = (640, 1024, 1152, 2048, 3072, 4096, 128, 384)
    Ms = (1, 2, 5, 16, 1, 3, 7, 1)
    items, refs = [], []
    for i in range(40):
        K, M = Ks[i % len(Ks)], Ms[(i // 3) % len(Ms)]
        N = 3072 if i % 5 else 1000
        x, nw, packed, scale = proj_inputs(19, i, 0, M, K, N, heavy=(i % 4 == 1))
        if M > 2:
            x[M - 1] = 0.0
        it = dict(x=dev(x), norm_w=dev(nw), packed_w=dev(packed), w_scale=scale, eps=EPS, N=N,
                  y=torch.full((M, N), float("nan"), device=DEV))
        items.append(it)
        refs.append((x, nw, packed, N))
    singles = [bl.bitlinear_forward(it["x"], it["norm_w"], it["packed_w"], it["w_scale"], it["N"], EPS)
               for it in items]
    with bl.Group(items) as g:
        g.forward()
        torch.cuda.synchronize()
        for it, ys in zip(items, singles):
            assert torch.equal(it["y"], ys)
    for i in (0, 7, 13, 22, 39):
        x, nw, packed, N = refs[i]
        assert rel_l2(host(singles[i]), oracle.bitlinear(x, nw, packed, N, EPS)) <= 1e-3


def test_determinism_nan_poison_and_guards():
    for M in (8, 600):
        K, N = 2048, 1000
        x, nw, packed, scale = proj_inputs(16, M, 0, M, K, N)
        dx, dn, dp = dev(x), dev(nw), dev(packed)
        guard = 4096
        buf = torch.full((M * N + 2 * guard,), float("nan"), device=DEV)
        y = buf[guard:guard + M * N].view(M, N)
        bl.bitlinear_forward(dx, dn, dp, scale, N, EPS, y=y)
        y1 = host(y).copy()
        assert np.all(np.isfinite(y1)), "unwritten output elements"
        b = host(buf)
        assert np.all(np.isnan(b[:guard])) and np.all(np.isnan(b[guard + M * N:])), "write outside y"
        y.fill_(float("nan"))
        bl.bitlinear_forward(dx, dn, dp, scale, N, EPS, y=y)
        assert np.array_equal(host(y), y1), "two runs differ"


def test_group_matches_separate_calls():
    items, singles = [], []
    for wid in (2, 3, 1):
        w = inputs.WORKLOADS[wid]
        for pi, (name, K, N) in enumerate(w.projs):
            x, nw, packed, scale = proj_inputs(wid, 0, pi, w.M, K, N)
            it = dict(x=dev(x), norm_w=dev(nw), packed_w=dev(packed), w_scale=scale, eps=EPS, N=N,
                      y=torch.full((w.M, N), float("nan"), device=DEV))
            items.append(it)
            singles.append(bl.bitlinear_forward(it["x"], it["norm_w"], it["packed_w"], scale, N, EPS))
    with bl.Group(items) as g:
        g.forward()
        torch.cuda.synchronize()
        for it, ys in zip(items, singles):
            assert torch.equal(it["y"], ys)
        for it in items:
            it["y"].fill_(float("nan"))
        g.quant()
        g.matmul()
        torch.cuda.synchronize()
        for it, ys in zip(items, singles):
            assert torch.equal(it["y"], ys)
        # The matmul stage launch by launch: the fused M = 1 problems (K 1024,
        # 2048, 3072 -> 4, 8, 12 superblocks) in one merged launch, the M = 8
        # problem unfused (its fp32 rows exceed the on-chip staging), then
        # prefill.
        info = g.launches()
        assert [d["kind"] for d in info] == ["decode_fused", "decode", "prefill"]
        assert [d["bucket"] for d in info[:2]] == [0, 4]
        assert info[0]["count"] == 7
        assert sum(d["count"] for d in info) == len(items)
        for it in items:
            it["y"].fill_(float("nan"))
        g.quant()
        for i in range(len(info)):
            g.matmul_launch(i)
        torch.cuda.synchronize()
        for it, ys in zip(items, singles):
            assert torch.equal(it["y"], ys)


@pytest.mark.parametrize("M", [300, 2304])
def test_group_shared_input_quantization(M):
    # Projections reading one x (q/k/v-like, gate/up-like) share a pass of
    # the quantization launch; a projection on the same x with another eps,
    # or on a prefix view of x with another M, must not join the set.  At
    # M = 300 the group's quantization is one merged launch; at M = 2304 it
    # needs more than 2048 workgroups, so the classes launch separately.
    x = dev(inputs.activations(21, 0, 0, M, 1024))
    x2 = dev(inputs.activations(21, 0, 1, M, 2048))
    specs = [(x, 1024, 512, EPS), (x, 1024, 256, EPS), (x2, 2048, 384, EPS), (x, 1024, 128, EPS),
             (x, 1024, 96, 1e-3), (x[:M - 37], 1024, 64, EPS), (x2, 2048, 200, EPS)]
    items, singles = [], []
    for i, (xx, K, N, eps) in enumerate(specs):
        W = inputs.weight(21, 1, i, N, K)
        packed, scale = oracle.i2s_pack(W)
        nw = dev(inputs.norm_weight(21, 1, i, K))
        it = dict(x=xx, norm_w=nw, packed_w=dev(packed), w_scale=scale, eps=eps, N=N,
                  y=torch.full((xx.shape[0], N), float("nan"), device=DEV))
        items.append(it)
        singles.append(bl.bitlinear_forward(xx, nw, it["packed_w"], scale, N, eps))
    with bl.Group(items) as g:
        info = g.forward_launches()
        if M == 300:
            assert (info[0]["kind"], info[0]["bucket"], info[0]["count"]) == ("quant_merged", 0, 7)
            assert not any(d["kind"].startswith("quant") for d in info[1:])
        else:
            assert [(d["kind"], d["bucket"], d["count"]) for d in info[:3]] == [
                ("quant", 4, 2), ("quant_shared", 4, 3), ("quant_shared", 8, 2)]
        g.forward()
        torch.cuda.synchronize()
        for i, (it, ys) in enumerate(zip(items, singles)):
            assert torch.equal(it["y"], ys), i
    # and against the oracle for one member of each set
    for i in (0, 2, 3, 6):
        xx, K, N, eps = specs[i]
        W = inputs.weight(21, 1, i, N, K)
        packed, _ = oracle.i2s_pack(W)
        ref = oracle.bitlinear(host(xx), inputs.norm_weight(21, 1, i, K), packed, N, eps)
        assert rel_l2(host(items[i]["y"]), ref) <= 1e-3


@pytest.mark.parametrize("M", [260, 2304])
def test_group_large_share_sets_split(M):
    # Share sets larger than the register-resident share kernel holds (3
    # problems at K <= 1024, 2 at K = 2048) are split; every part still reads
    # x once and gives bit-identical results to separate calls, with norm
    # weights of every kind (float32, float16, none) inside one set.  At
    # M = 260 the parts run in one merged launch, at M = 2304 in launches per
    # class.
    x = dev(inputs.activations(27, 0, 0, M, 1024))
    x2 = dev(inputs.activations(27, 0, 1, M, 2048))
    specs = [(x, 1024, 64 * (i + 1), ("f32", "f16", "none")[i % 3]) for i in range(6)] + \
            [(x2, 2048, 96 * (i + 1), ("f32", "none", "f16")[i]) for i in range(3)]
    items, singles = [], []
    for i, (xx, K, N, kind) in enumerate(specs):
        packed, scale = oracle.i2s_pack(inputs.weight(27, 1, i, N, K))
        nw = dev(inputs.norm_weight(27, 1, i, K))
        nw = None if kind == "none" else (nw.half() if kind == "f16" else nw)
        it = dict(x=xx, norm_w=nw, packed_w=dev(packed), w_scale=scale, eps=EPS, N=N,
                  y=torch.full((M, N), float("nan"), device=DEV))
        items.append(it)
        singles.append(bl.bitlinear_forward(xx, nw, it["packed_w"], scale, N, EPS))
    with bl.Group(items) as g:
        q = sorted((d["kind"], d["bucket"], d["count"]) for d in g.forward_launches()
                   if d["kind"].startswith("quant"))
        # K = 1024: two parts of 3, one launch; K = 2048: a part of 2 and a single
        if M == 260:
            assert q == [("quant_merged", 0, 9)], q
        else:
            assert q == [("quant", 8, 1), ("quant_shared", 4, 6), ("quant_shared", 8, 2)], q
        g.forward()
        torch.cuda.synchronize()
        for i, (it, ys) in enumerate(zip(items, singles)):
            assert torch.equal(it["y"], ys), i


def test_group_forward_in_cuda_graph():
    # The group forward captured into a graph: the fused decode launches (the
    # merged one and a 13-superblock one, which stays separate) fork onto the
    # group's own streams and join back inside the capture.  Every replay
    # (eager work and synchronisation between replays) must reproduce
    # separate forward calls bit for bit.
    items, singles = [], []
    specs = [(1, 1024, 2048), (1, 2048, 1024), (1, 3072, 1024), (2, 640, 256), (8, 1024, 96),
             (20, 1024, 160), (1, 3328, 520)]
    for i, (M, K, N) in enumerate(specs):
        x, nw, packed, scale = proj_inputs(19, i, 0, M, K, N)
        it = dict(x=dev(x), norm_w=dev(nw), packed_w=dev(packed), w_scale=scale, eps=EPS, N=N,
                  y=torch.full((M, N), float("nan"), device=DEV))
        items.append(it)
        singles.append(bl.bitlinear_forward(it["x"], it["norm_w"], it["packed_w"], scale, N, EPS))
    with bl.Group(items) as g:
        kinds = [d["kind"] for d in g.forward_launches()]
        assert kinds.count("decode_fused") == 2 and "quant" in kinds and "prefill" in kinds
        g.forward()  # warm-up outside the capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            g.forward()
        for rep in range(3):
            for it in items:
                it["y"].fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for it, ys in zip(items, singles):
                assert torch.equal(it["y"], ys), f"replay {rep}"


def test_group_merged_decode_mixed_shapes():
    # Fused decode problems of very different M and K in one merged launch
    # (M = 16 at K = 256 beside M = 1 and 2 at K = 3072): the launch's LDS is
    # the largest single problem's staging, each workgroup lays its own out.
    # K = 4096 (16 superblocks) fuses in its own launch.
    nan = float("nan")
    items, singles = [], []
    for i, (M, K, N) in enumerate([(16, 256, 64), (1, 3072, 1024), (7, 1024, 200), (2, 3072, 96),
                                   (1, 4096, 80), (5, 2048, 48)]):
        x, nw, packed, scale = proj_inputs(32, i, 0, M, K, N)
        it = dict(x=dev(x), norm_w=dev(nw), packed_w=dev(packed), w_scale=scale, eps=EPS, N=N,
                  y=torch.full((M, N), nan, device=DEV))
        items.append(it)
        singles.append(bl.bitlinear_forward(it["x"], it["norm_w"], it["packed_w"], scale, N, EPS))
        if i == 0:
            assert rel_l2(host(singles[-1]), oracle.bitlinear(x, nw, packed, N, EPS)) <= 1e-3
    with bl.Group(items) as g:
        info = g.forward_launches()
        assert [(d["kind"], d["bucket"], d["count"]) for d in info] == [
            ("quant", 8, 1), ("decode_fused", 0, 4), ("decode", 8, 1), ("decode_fused", 16, 1)], info
        g.forward()
        torch.cuda.synchronize()
        for i, (it, ys) in enumerate(zip(items, singles)):
            assert torch.equal(it["y"], ys), i


def test_group_with_glue_in_cuda_graph():
    # A group with FFN-glue descriptors (fused glue decode, glue quantization
    # for an unfused decode and a prefill problem) beside a plain fused one,
    # captured into a graph; every replay equals the single calls bit for bit.
    nan = float("nan")
    items, singles = [], []
    for i, (act, M, K, N) in enumerate([(bl.ACT_SILU, 1, 3072, 1024), (bl.ACT_GELU_TANH, 8, 2048, 640),
                                        (bl.ACT_SILU, 40, 1024, 160)]):
        gate, up, nw, packed, scale = glu_inputs(act, M, K, N, seed=30 + i)
        it = dict(x=dev(gate), up=dev(up), act=act, norm_w=dev(nw), packed_w=dev(packed), w_scale=scale,
                  eps=EPS, N=N, y=torch.full((M, N), nan, device=DEV))
        items.append(it)
        singles.append(bl.bitlinear_glu_forward(it["x"], it["up"], act, it["norm_w"], it["packed_w"],
                                                scale, N, EPS))
    x, nw, packed, scale = proj_inputs(31, 0, 0, 1, 1024, 512)
    it = dict(x=dev(x), norm_w=dev(nw), packed_w=dev(packed), w_scale=scale, eps=EPS, N=512,
              y=torch.full((1, 512), nan, device=DEV))
    items.append(it)
    singles.append(bl.bitlinear_forward(it["x"], it["norm_w"], it["packed_w"], scale, 512, EPS))
    with bl.Group(items) as g:
        kinds = [d["kind"] for d in g.forward_launches()]
        assert kinds == ["quant_glue", "quant_glue", "decode_fused", "decode", "decode_fused_glue",
                         "prefill"], kinds
        g.forward()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            g.forward()
        for rep in range(3):
            for it in items:
                it["y"].fill_(nan)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for i, (it, ys) in enumerate(zip(items, singles)):
                assert torch.equal(it["y"], ys), (rep, i)


# ------------------------------------------------------------ no norm ---
# A projection without its own norm weight ("BitNet Embeddings GGUF
# Conversion Implementation", s4.5: the shared input feeds the projection
# directly): norm_w NULL, codes from max|x|, factor max|x|/127.  Every
# quantization variant (register, shared, streaming, fused decode) takes it.

NO_NORM_QUANT_CASES = [(1, 128), (8, 1024), (300, 3072), (7, 4096), (257, 640), (3, 8192)]


@pytest.mark.parametrize("M,K", NO_NORM_QUANT_CASES)
def test_no_norm_quant_parity(M, K):
    x = inputs.activations(23, 0, K, M, K, heavy_tail=True)
    if M > 3:
        x[1] = 0.0
        x[2] *= 1e-36
    xq, f = bl.bitlinear_quant(dev(x), None, EPS)
    q_ref, f_ref = oracle.quant(x, None, EPS)
    flips = check_codes(host(xq), q_ref, x, np.ones(K, np.float32))
    # max|x| is exact in fp32, so the factor is the correctly rounded max|x|/127
    assert np.array_equal(host(f), f_ref.astype(np.float32))
    log(f"no-norm quant M={M} K={K}: {flips} flips")


NO_NORM_FWD_CASES = [(1, 1024, 3072), (4, 2048, 640), (16, 3072, 96), (16, 4096, 48),
                     (17, 2048, 640), (300, 1024, 1024), (5, 8192, 130)]


@pytest.mark.parametrize("M,K,N", NO_NORM_FWD_CASES)
def test_no_norm_forward_parity_and_hooks(M, K, N):
    # decode fused (small M*K), decode unfused, prefill and the streaming
    # quantization (K 8192); forward == fp32 epilogue of matmul_i32 o quant.
    x, _, packed, scale = proj_inputs(23, 1, K, M, K, N, heavy=True)
    if M > 2:
        x[M // 2] = 0.0
    dx, dp = dev(x), dev(packed)
    y = bl.bitlinear_forward(dx, None, dp, scale, N, EPS)
    ref = oracle.bitlinear(x, None, packed, N, EPS)
    assert rel_l2(host(y), ref) <= 1e-3
    if M > 2:
        assert not np.any(host(y)[M // 2])
    xq, f = bl.bitlinear_quant(dx, None, EPS)
    acc = bl.bitlinear_matmul_i32(xq, dp, N)
    y2 = acc.to(torch.float32) * (f / torch.tensor(scale, dtype=torch.float32, device=DEV))[:, None]
    assert torch.equal(y, y2)


def test_no_norm_group_mixed_with_normed_share_set():
    # One x read by projections with and without a norm weight: they share
    # the quantization pass (and, at M <= 16, the fused decode), each with its
    # own arithmetic; results equal separate calls bit for bit.
    items, singles = [], []
    for M in (1, 8, 300):
        for K in (1024, 3072):
            x = dev(inputs.activations(24, M, K, M, K))
            for i, N in enumerate((256, 128, 96)):
                W = inputs.weight(24, M, K + i, N, K)
                packed, scale = oracle.i2s_pack(W)
                nw = None if i == 1 else dev(inputs.norm_weight(24, M, K + i, K))
                it = dict(x=x, norm_w=nw, packed_w=dev(packed), w_scale=scale, eps=EPS, N=N,
                          y=torch.full((M, N), float("nan"), device=DEV))
                items.append(it)
                singles.append(bl.bitlinear_forward(x, nw, it["packed_w"], scale, N, EPS))
    with bl.Group(items) as g:
        kinds = [d["kind"] for d in g.forward_launches()]
        # share sets at K = 1024, single problems at K = 3072 (12 chunks): one
        # merged quantization launch for this small group
        assert "quant_merged" in kinds and "decode_fused" in kinds
        g.forward()
        torch.cuda.synchronize()
        for i, (it, ys) in enumerate(zip(items, singles)):
            assert torch.equal(it["y"], ys), i
    it = items[-2]  # M 300, K 3072, no norm
    W = inputs.weight(24, 300, 3072 + 1, 128, 3072)
    packed, _ = oracle.i2s_pack(W)
    assert rel_l2(host(it["y"]), oracle.bitlinear(host(it["x"]), None, packed, 128, EPS)) <= 1e-3


@pytest.mark.parametrize("act,M,K,N", [(bl.ACT_SILU, 1, 3072, 1024), (bl.ACT_GELU_TANH, 2, 2048, 640),
                                       (bl.ACT_GELU_TANH, 300, 2048, 640)])
def test_no_norm_glu_forward(act, M, K, N):
    gate, up, _, packed, scale = glu_inputs(act, M, K, N, seed=2)
    y = bl.bitlinear_glu_forward(dev(gate), dev(up), act, None, dev(packed), scale, N, EPS)
    assert rel_l2(host(y), oracle.glu_bitlinear(gate, up, act, None, packed, N, EPS)) <= 1e-3
    xq, f = bl.bitlinear_glu_quant(dev(gate), dev(up), act, None, EPS)
    q_ref, f_ref = oracle.glu_quant(gate, up, act, None, EPS)
    check_codes(host(xq), q_ref, oracle.glu(gate, up, act), np.ones(K, np.float32))
    check_factor(host(f), f_ref)


# ------------------------------------------------------ f16 norm weights ---
# Norm weights stored as float16 ("BitNet Embeddings GGUF Conversion
# Implementation", s3 tensor type table, s6.1): widened exactly on load, so
# every result equals the float32 path on the widened weights bit for bit,
# and the oracle's float16 path within the usual criteria.

F16_CASES = [(1, 1024, 3072), (4, 640, 96), (16, 3072, 96), (8, 4096, 48), (17, 2048, 640),
             (300, 1024, 1024), (5, 8192, 130), (257, 3072, 64)]


@pytest.mark.parametrize("M,K,N", F16_CASES)
def test_f16_norm_weight_equals_widened_f32(M, K, N):
    # fused decode (M*K small), unfused decode, prefill, streaming (K 8192)
    x, nw, packed, scale = proj_inputs(26, M, K, M, K, N, heavy=True)
    if M > 2:
        x[M // 2] = 0.0
    nw16 = nw.astype(np.float16)
    dx, dp = dev(x), dev(packed)
    d16 = torch.from_numpy(nw16).to(DEV)
    dwide = dev(nw16.astype(np.float32))
    y16 = bl.bitlinear_forward(dx, d16, dp, scale, N, EPS)
    y32 = bl.bitlinear_forward(dx, dwide, dp, scale, N, EPS)
    assert torch.equal(y16, y32)
    q16, f16 = bl.bitlinear_quant(dx, d16, EPS)
    q32, f32 = bl.bitlinear_quant(dx, dwide, EPS)
    assert torch.equal(q16, q32) and torch.equal(f16, f32)
    assert rel_l2(host(y16), oracle.bitlinear(x, nw16, packed, N, EPS)) <= 1e-3
    q_ref, f_ref = oracle.quant(x, nw16, EPS)
    check_codes(host(q16), q_ref, x, nw16.astype(np.float32))
    check_factor(host(f16), f_ref)


def test_f16_norm_weight_group_mixed_kinds():
    # One x read by projections with float32, float16 and no norm weights, in
    # share sets and fused decode launches: equal to separate calls.
    items, singles = [], []
    for M in (1, 8, 300):
        x = dev(inputs.activations(27, M, 0, M, 1024))
        for i, N in enumerate((256, 128, 96, 64)):
            W = inputs.weight(27, M, i, N, 1024)
            packed, scale = oracle.i2s_pack(W)
            nw = inputs.norm_weight(27, M, i, 1024)
            nw = [dev(nw), torch.from_numpy(nw.astype(np.float16)).to(DEV), None,
                  torch.from_numpy(nw.astype(np.float16)).to(DEV)][i]
            it = dict(x=x, norm_w=nw, packed_w=dev(packed), w_scale=scale, eps=EPS, N=N,
                      y=torch.full((M, N), float("nan"), device=DEV))
            items.append(it)
            singles.append(bl.bitlinear_forward(x, nw, it["packed_w"], scale, N, EPS))
    with bl.Group(items) as g:
        kinds = [d["kind"] for d in g.forward_launches()]
        # a set of 3 and a single at M = 300: one merged quantization launch
        assert "quant_merged" in kinds and "decode_fused" in kinds and "prefill" in kinds
        g.forward()
        torch.cuda.synchronize()
        for i, (it, ys) in enumerate(zip(items, singles)):
            assert torch.equal(it["y"], ys), i


@pytest.mark.parametrize("act,M,K,N", [(bl.ACT_SILU, 1, 3072, 1024), (bl.ACT_GELU_TANH, 300, 2048, 640),
                                       (bl.ACT_SILU, 6, 8192, 96)])
def test_f16_norm_weight_glu(act, M, K, N):
    gate, up, nw, packed, scale = glu_inputs(act, M, K, N, seed=3)
    nw16 = nw.astype(np.float16)
    dg, du, dp = dev(gate), dev(up), dev(packed)
    d16, dwide = torch.from_numpy(nw16).to(DEV), dev(nw16.astype(np.float32))
    y16 = bl.bitlinear_glu_forward(dg, du, act, d16, dp, scale, N, EPS)
    assert torch.equal(y16, bl.bitlinear_glu_forward(dg, du, act, dwide, dp, scale, N, EPS))
    q16, f16 = bl.bitlinear_glu_quant(dg, du, act, d16, EPS)
    q32, f32 = bl.bitlinear_glu_quant(dg, du, act, dwide, EPS)
    assert torch.equal(q16, q32) and torch.equal(f16, f32)
    assert rel_l2(host(y16), oracle.glu_bitlinear(gate, up, act, nw16, packed, N, EPS)) <= 1e-3


# ---------------------------------------------------------------- FFN glue ---
# The down projection fed by act(gate) * up ("BitNet Embeddings GGUF
# Conversion Implementation", s4.5 FFN per-projection norms): the GPU forms
# the product in fp32 registers, the oracle in double; codes and outputs meet
# the same criteria as the plain path.

def glu_inputs(act, M, K, N=None, seed=0):
    gate = inputs.activations(22, seed, 2 * act, M, K) * np.float32(2.0)
    up = inputs.activations(22, seed, 2 * act + 1, M, K)
    nw = inputs.norm_weight(22, seed, act, K)
    if M > 3:
        gate[1] = 0.0               # zero product: zero codes, factor 0
        gate[2] = -20.0             # activation ~0 but not 0: a tiny row
        up[3] = 0.0
    out = [gate, up, nw]
    if N is not None:
        W = inputs.weight(22, seed, act, N, K)
        packed, scale = oracle.i2s_pack(W)
        out += [packed, scale]
    return out


GLU_QUANT_CASES = [(act, M, K) for act in (bl.ACT_SILU, bl.ACT_GELU_TANH)
                   for M, K in ((1, 3072), (8, 2048), (300, 3072), (257, 640), (6, 8192))]


@pytest.mark.parametrize("act,M,K", GLU_QUANT_CASES)
def test_glu_quant_parity(act, M, K):
    gate, up, nw = glu_inputs(act, M, K)
    xq, f = bl.bitlinear_glu_quant(dev(gate), dev(up), act, dev(nw), EPS)
    q_ref, f_ref = oracle.glu_quant(gate, up, act, nw, EPS)
    h = oracle.glu(gate, up, act)
    flips = check_codes(host(xq), q_ref, h, nw)
    check_factor(host(f), f_ref)
    log(f"glu quant act={act} M={M} K={K}: {flips} code flips")


GLU_FWD_CASES = [(act, M, K, N) for act in (bl.ACT_SILU, bl.ACT_GELU_TANH)
                 for M, K, N in ((1, 3072, 1024), (2, 2048, 640), (3, 1024, 200), (4, 2048, 640),
                                 (16, 3072, 96), (17, 2048, 640), (512, 2048, 640), (300, 3072, 1024))]
# M = 1..3 at these K run the glue inside the one-launch fused decode; the
# hooks comparison below then checks it bit for bit against the two-stage path.


@pytest.mark.parametrize("act,M,K,N", GLU_FWD_CASES)
def test_glu_forward_parity_and_hooks(act, M, K, N):
    gate, up, nw, packed, scale = glu_inputs(act, M, K, N, seed=1)
    dg, du, dn, dp = dev(gate), dev(up), dev(nw), dev(packed)
    y = bl.bitlinear_glu_forward(dg, du, act, dn, dp, scale, N, EPS)
    ref = oracle.glu_bitlinear(gate, up, act, nw, packed, N, EPS)
    assert rel_l2(host(y), ref) <= 1e-3
    if M > 3:
        assert not np.any(host(y)[1])                  # the zero-product row
    # forward == fp32 epilogue of matmul_i32 o glu_quant, bit for bit
    xq, f = bl.bitlinear_glu_quant(dg, du, act, dn, EPS)
    acc = bl.bitlinear_matmul_i32(xq, dp, N)
    y2 = acc.to(torch.float32) * (f / torch.tensor(scale, dtype=torch.float32, device=DEV))[:, None]
    assert torch.equal(y, y2)


def test_group_ffn_glue_descriptors():
    # Glue descriptors in a group beside plain ones: fused decode with the glue
    # (M = 1, K = 3072, SiLU; M = 2, K = 2048, GELU-tanh), unfused decode
    # (M = 8), prefill (M = 300), a fused plain M = 1 problem and a plain pair
    # sharing its input.  Every output equals its single call bit for bit.
    nan = float("nan")
    items, singles = [], []
    for i, (act, M, K, N) in enumerate([(bl.ACT_SILU, 1, 3072, 1024), (bl.ACT_GELU_TANH, 2, 2048, 640),
                                        (bl.ACT_SILU, 8, 2048, 640), (bl.ACT_GELU_TANH, 300, 3072, 200)]):
        gate, up, nw, packed, scale = glu_inputs(act, M, K, N, seed=20 + i)
        it = dict(x=dev(gate), up=dev(up), act=act, norm_w=dev(nw), packed_w=dev(packed), w_scale=scale,
                  eps=EPS, N=N, y=torch.full((M, N), nan, device=DEV))
        items.append(it)
        singles.append(bl.bitlinear_glu_forward(it["x"], it["up"], act, it["norm_w"], it["packed_w"],
                                                scale, N, EPS))
        if M in (2, 300):
            ref = oracle.glu_bitlinear(gate, up, act, nw, packed, N, EPS)
            assert rel_l2(host(singles[-1]), ref) <= 1e-3
    x1, nw1, p1, s1 = proj_inputs(21, 0, 0, 1, 1024, 256)
    x3, nw3, p3, s3 = proj_inputs(21, 1, 0, 300, 1024, 128)
    _, nw4, p4, s4 = proj_inputs(21, 1, 1, 300, 1024, 96)
    dx3 = dev(x3)
    for x, nw, packed, scale, N in ((dev(x1), nw1, p1, s1, 256), (dx3, nw3, p3, s3, 128), (dx3, nw4, p4, s4, 96)):
        it = dict(x=x, norm_w=dev(nw), packed_w=dev(packed), w_scale=scale, eps=EPS, N=N,
                  y=torch.full((x.shape[0], N), nan, device=DEV))
        items.append(it)
        singles.append(bl.bitlinear_forward(it["x"], it["norm_w"], it["packed_w"], scale, N, EPS))
    with bl.Group(items) as g:
        g.forward()
        torch.cuda.synchronize()
        for i, (it, ys) in enumerate(zip(items, singles)):
            assert torch.equal(it["y"], ys), i
        info = g.forward_launches()
        assert [d["kind"] for d in info] == ["quant_shared", "quant_glue", "quant_glue", "decode_fused",
                                            "decode", "decode_fused_glue", "decode_fused_glue", "prefill"]
        assert [d["bucket"] for d in info] == [4, 8, 12, 0, 8, 8, 12, 0]
        for it in items:
            it["y"].fill_(nan)
        for i in range(len(info)):
            g.forward_launch(i)
        torch.cuda.synchronize()
        for i, (it, ys) in enumerate(zip(items, singles)):
            assert torch.equal(it["y"], ys), i


def test_glu_forward_qwen_down_full_size_sampled_rows():
    # The Qwen3 FFN down projection at the long-context size (M = 32768,
    # K = 3072 -> N = 1024, SiLU), checked on sampled rows.
    act, M, K, N = bl.ACT_SILU, 32768, 3072, 1024
    dg = inputs.activations_device(torch, 22, 9, 0, M, K, DEV)
    du = inputs.activations_device(torch, 22, 9, 1, M, K, DEV)
    nw = inputs.norm_weight(22, 9, 0, K)
    W = inputs.weight(22, 9, 0, N, K)
    packed, scale = oracle.i2s_pack(W)
    y = bl.bitlinear_glu_forward(dg, du, act, dev(nw), dev(packed), scale, N, EPS)
    rows = inputs.sample_rows(M, 16, seed=9)
    idx = torch.as_tensor(rows, device=DEV)
    ref = oracle.glu_bitlinear(host(dg[idx]), host(du[idx]), act, nw, packed, N, EPS)
    assert rel_l2(host(y[idx]), ref) <= 1e-3


# ------------------------------------------ full-size workloads, sampled ---
# Workloads 4 and 5 run at full size in the grouped launch the bench times,
# into NaN-filled outputs (every element must be written: a skipped or
# mis-indexed tile would leave a NaN).  Each BitLinear is then checked on one
# seeded row in every 128-row tile of the prefill kernel (rows drawn per
# BitLinear), plus the first and the last row:
#   * the group's output equals the fp32 epilogue of the hooks
#     (matmul_i32 o quant) bit for bit;
#   * the int8 codes and factors meet the quantization criteria against the
#     oracle;
#   * for the BitLinears in `exact`, matmul_i32 fed the oracle's own codes of
#     the whole matrix equals the oracle's int32 product exactly;
#   * on a smaller per-BitLinear sample, rel L2 <= 1e-3 against the oracle.
# The oracle runs in host threads (its C functions release the GIL).

ORACLE_THREADS = 16
TILE_M = 128  # activation rows per prefill workgroup tile


def _pool_map(fn, jobs):
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(ORACLE_THREADS) as ex:
        return list(ex.map(fn, jobs))


def _full_size_checks(items, refs, exact, l2_rows):
    """items: group dicts (y NaN-filled); refs: (x host, norm_w, packed, scale,
    N, tag, seed) per item; exact: indices of items whose int32 product is
    compared with the oracle on every tile row."""
    with bl.Group(items) as g:
        g.forward()
        torch.cuda.synchronize()
    flips = codes = 0
    l2_jobs, exact_jobs = [], []
    for i, (it, (x, nw, packed, scale, N, tag, seed)) in enumerate(zip(items, refs)):
        M, K = x.shape
        y = it["y"]
        assert bool(torch.isfinite(y).all()), f"{tag}: output elements left unwritten"
        rows = inputs.tile_rows(M, TILE_M, seed)
        assert len(np.unique(rows // TILE_M)) == (M + TILE_M - 1) // TILE_M
        idx = torch.as_tensor(rows, device=DEV)
        xq, f = bl.bitlinear_quant(it["x"], it["norm_w"], EPS)
        acc = bl.bitlinear_matmul_i32(xq, it["packed_w"], N)
        assert torch.equal(y[idx], _hooks_epilogue(acc[idx], f[idx], scale)), \
            f"{tag}: group output differs from the hooks' composition"
        q_ref, f_ref = oracle.quant(x[rows], nw, EPS)
        flips += check_codes(host(xq[idx]), q_ref, x[rows], nw)
        codes += q_ref.size
        check_factor(host(f[idx]), f_ref)
        del xq, acc
        lrows = inputs.sample_rows(M, l2_rows, seed=seed)
        l2_jobs.append((host(y[torch.as_tensor(lrows, device=DEV)]), x[lrows], nw, packed, N, tag))
        if i in exact:
            q_all, _ = oracle.quant(x, nw, EPS)
            acc_o = bl.bitlinear_matmul_i32(dev(q_all), it["packed_w"], N)
            exact_jobs.append((host(acc_o[idx]), q_all[rows], packed, K, N, tag))
            del acc_o

    def l2(job):
        y_gpu, xr, nw, packed, N, tag = job
        return rel_l2(y_gpu, oracle.bitlinear(xr, nw, packed, N, EPS)), tag

    def exact_eq(job):
        acc_gpu, qr, packed, K, N, tag = job
        return np.array_equal(acc_gpu, oracle.matmul_i32(qr, packed, K, N)), tag

    worst = 0.0
    for err, tag in _pool_map(l2, l2_jobs):
        assert err <= 1e-3, f"{tag}: rel L2 {err}"
        worst = max(worst, err)
    for ok, tag in _pool_map(exact_eq, exact_jobs):
        assert ok, f"{tag}: int32 product differs from the oracle's"
    assert flips <= 1e-4 * codes, f"{flips} code flips in {codes}"
    return worst, flips, codes


def test_workload4_full_size_sampled_rows():
    w = inputs.WORKLOADS[4]
    xs = {}
    for pi, (name, K, N) in enumerate(w.projs):
        if K not in xs:
            x = inputs.activations(4, 0, K, w.M, K)
            xs[K] = (x, dev(x))
    items, refs = [], []
    for layer in range(w.layers):
        for pi, (name, K, N) in enumerate(w.projs):
            W = inputs.weight(4, layer, pi, N, K)
            packed, scale = oracle.i2s_pack(W)
            nw = inputs.norm_weight(4, layer, pi, K)
            items.append(dict(x=xs[K][1], norm_w=dev(nw), packed_w=dev(packed), w_scale=scale,
                              eps=EPS, N=N, y=torch.full((w.M, N), float("nan"), device=DEV)))
            refs.append((xs[K][0], nw, packed, scale, N, f"layer {layer} {name}", 100 * layer + pi))
        if layer % 7 == 6:
            log(f"workload 4: layers 0..{layer} prepared")
    exact = set(range(len(w.projs))) | set(range(len(items) - len(w.projs), len(items)))
    worst, flips, codes = _full_size_checks(items, refs, exact, 8)
    log(f"workload 4: worst rel L2 {worst:.2e}, {flips} code flips in {codes}")


def test_workload5_full_size_sampled_rows():
    w = inputs.WORKLOADS[5]
    items, refs = [], []
    for pi, (name, K, N) in enumerate(w.projs):
        x, nw, packed, scale = proj_inputs(5, 0, pi, w.M, K, N, heavy=True)
        items.append(dict(x=dev(x), norm_w=dev(nw), packed_w=dev(packed), w_scale=scale, eps=EPS,
                          N=N, y=torch.full((w.M, N), float("nan"), device=DEV)))
        refs.append((x, nw, packed, scale, N, name, 500 + pi))
    worst, flips, codes = _full_size_checks(items, refs, set(range(len(items))), 16)
    log(f"workload 5: worst rel L2 {worst:.2e}, {flips} code flips in {codes}")


# ------------------------------------------------------- device-side packing ---
# i2s_pack_device against the oracle's packing: the same bytes and the same
# float32 scale (the byte layout is pinned in the oracle's own tests).

def _pack_dev_check(W, tag):
    packed, scale = bl.i2s_pack_device(dev(W))
    p_ref, s_ref = oracle.i2s_pack(W)
    assert scale == s_ref, f"{tag}: scale {scale} vs {s_ref}"
    assert np.array_equal(host(packed), p_ref), f"{tag}: bytes differ"
    return packed, scale


def test_pack_device_worked_examples():
    pat = np.array([0.5, -0.5, 0.125, -0.125, 0.375, -0.0625, 0.1875, -0.125], np.float32)
    W = np.stack([np.tile(pat, 16), -np.tile(pat, 16)])
    packed, scale = _pack_dev_check(W, "W1")
    assert scale == 4.0 and host(packed)[:8].tolist() == [0xAA, 0x00, 0x55, 0x55, 0xAA, 0x55, 0xAA, 0x55]
    # one-hot rows at every position of a block: mean|W| = 1/128, scale 128
    _pack_dev_check(np.eye(128, dtype=np.float32), "one-hot family")
    _pack_dev_check(np.zeros((3, 256), np.float32), "all zero")


SHAPES_DEV = sorted({(N, K) for w in inputs.WORKLOADS.values() for (_, K, N) in w.projs})


@pytest.mark.parametrize("N,K", SHAPES_DEV)
def test_pack_device_workload_shapes(N, K):
    _pack_dev_check(inputs.weight(8, 0, K + N, N, K), f"N={N} K={K}")


@pytest.mark.parametrize("N,K", [(1, 128), (3, 8192), (7, 384), (4099, 256), (3072, 3072)])
def test_pack_device_ragged_and_large(N, K):
    W = inputs.weight(8, 2, N, N, K)
    W[::5, ::3] = 0.0
    _pack_dev_check(W, f"N={N} K={K}")


def test_pack_device_ties_and_determinism():
    ties = np.tile(np.array([0.5, -0.5, 1.5, -1.5, 2.5, 0.25, -0.25, 1.0], np.float32), 16)
    _pack_dev_check(np.stack([ties, ties * 2, -ties]), "ties")
    W = dev(inputs.weight(8, 3, 0, 1024, 1280))
    a, sa = bl.i2s_pack_device(W)
    b, sb = bl.i2s_pack_device(W)
    assert sa == sb and torch.equal(a, b)


def test_pack_device_async_tail_and_nonfinite():
    W = inputs.weight(8, 4, 0, 256, 1024)
    packed, scale = bl.i2s_pack_device(dev(W), read_scale=False)
    assert scale is None
    p_ref, s_ref = oracle.i2s_pack(W)
    got = host(packed)
    assert np.array_equal(got, p_ref)
    assert got[-4:].view(np.float32)[0] == s_ref
    for bad in (np.nan, np.inf, -np.inf):
        Wb = W.copy()
        Wb[17, 5] = bad
        with pytest.raises(bl.BitLinearError) as e:
            bl.i2s_pack_device(dev(Wb))
        assert e.value.status == bl.BL_ERR_NONFINITE


def test_forward_with_device_packed_weights():
    M, K, N = 300, 1024, 640
    W = inputs.weight(8, 5, 0, N, K)
    x = inputs.activations(8, 5, 0, M, K)
    nw = inputs.norm_weight(8, 5, 0, K)
    pd, sd = bl.i2s_pack_device(dev(W))
    ph, sh = oracle.i2s_pack(W)
    y_d = host(bl.bitlinear_forward(dev(x), dev(nw), pd, sd, N, EPS))
    y_h = host(bl.bitlinear_forward(dev(x), dev(nw), dev(ph), sh, N, EPS))
    assert np.array_equal(y_d, y_h)
    assert rel_l2(y_d, oracle.bitlinear(x, nw, ph, N, EPS)) <= 1e-3


# ------------------------------------------------- stateless batched call ---

def _mixed_items(seed, specs):
    """Group-style items over (M, K, N, kind) specs; kind: "plain", "nonorm",
    "f16", "glu" (SiLU glue) or "shared" (reads the previous item's x)."""
    items = []
    for i, (M, K, N, kind) in enumerate(specs):
        x, nw, packed, scale = proj_inputs(seed, i, 0, M, K, N)
        it = dict(x=dev(x), norm_w=dev(nw), packed_w=dev(packed), w_scale=scale, eps=EPS, N=N,
                  y=torch.full((M, N), float("nan"), device=DEV))
        if kind == "nonorm":
            it["norm_w"] = None
        elif kind == "f16":
            it["norm_w"] = it["norm_w"].half()
        elif kind == "glu":
            it["up"] = dev(inputs.activations(seed, i, 1, M, K))
            it["act"] = bl.ACT_SILU
        elif kind == "shared":
            it["x"] = items[-1]["x"]
        items.append(it)
    return items


def _single(it):
    if "up" in it:
        return bl.bitlinear_glu_forward(it["x"], it["up"], it["act"], it["norm_w"], it["packed_w"],
                                        it["w_scale"], it["N"], EPS)
    return bl.bitlinear_forward(it["x"], it["norm_w"], it["packed_w"], it["w_scale"], it["N"], EPS)


def test_batched_matches_separate_calls():
    # Decode (fused, unfused, long rows), prefill, shared inputs, glue, no
    # norm and float16 norms in one stateless call; then a smaller and a
    # larger call on the same stream (the second grows the workspace).
    specs = [(1, 1024, 2048, "plain"), (1, 1024, 1024, "shared"), (1, 3072, 1024, "glu"),
             (8, 1024, 96, "plain"), (16, 8192, 40, "nonorm"), (300, 2048, 640, "plain"),
             (300, 2048, 640, "shared"), (40, 640, 256, "f16"), (17, 3072, 100, "glu"),
             (3, 640, 33, "nonorm"), (0, 1024, 64, "plain")]
    for seed, sp in ((25, specs), (26, specs[:4]), (27, specs + [(2048, 3072, 1024, "plain")])):
        items = _mixed_items(seed, sp)
        bl.bitlinear_forward_batched(items)
        torch.cuda.synchronize()
        for it in items:
            if it["x"].shape[0]:
                assert torch.equal(it["y"], _single(it)), (seed, it["x"].shape, it["N"])
        log(f"batched seed {seed}: {len(items)} descriptors bit-identical to single calls")
    # checked once against the oracle as well
    x, nw, packed, scale = proj_inputs(27, 5, 0, 300, 2048, 640)
    assert rel_l2(host(items[5]["y"]), oracle.bitlinear(x, nw, packed, 640, EPS)) <= 1e-3


SPLIT_GROUPS = [
    # The Gemma3-270M layer at M = 512 (q, k, v and gate, up sharing x): o is
    # split 2 ways and down 4 ways on a 256-CU device.
    [(512, 640, 1024, "plain"), (512, 640, 256, "shared"), (512, 640, 256, "shared"),
     (512, 1024, 640, "plain"), (512, 640, 2048, "plain"), (512, 640, 2048, "shared"),
     (512, 2048, 640, "plain")],
    # Ragged rows and columns, uneven block splits (K = 3200: 25 blocks),
    # float16 and no norm weights, a decode problem beside them.
    [(300, 4096, 256, "plain"), (17, 3200, 520, "f16"), (129, 1536, 100, "nonorm"),
     (1, 1024, 64, "plain"), (40, 6272, 32, "plain")],
]


@pytest.mark.parametrize("gi", range(len(SPLIT_GROUPS)))
def test_group_split_prefill(gi):
    # Split prefill tiles (partial int32 tiles added by the last split to
    # arrive) against single calls, which never split: bit for bit, over
    # repeated forwards (the tile counts must come back to zero) and over
    # replays of a captured forward.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    items = _mixed_items(40 + gi, SPLIT_GROUPS[gi])
    splits = bl.prefill_splits(items, cus)
    log(f"split group {gi}: splits {splits} on {cus} CUs")
    assert max(splits) > 1
    singles = [_single(it) for it in items]
    with bl.Group(items) as g:
        for rep in range(4):
            for it in items:
                it["y"].fill_(float("nan"))
            g.forward()
            torch.cuda.synchronize()
            for i, (it, ys) in enumerate(zip(items, singles)):
                assert torch.equal(it["y"], ys), (gi, rep, i)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            g.forward()
        for rep in range(3):
            for it in items:
                it["y"].fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for i, (it, ys) in enumerate(zip(items, singles)):
                assert torch.equal(it["y"], ys), (gi, "replay", rep, i)
    # the most-split problem against the oracle as well
    i = int(np.argmax(splits))
    M, K, N, kind = SPLIT_GROUPS[gi][i]
    assert kind == "plain"
    x, nw, packed, scale = proj_inputs(40 + gi, i, 0, M, K, N)
    assert rel_l2(host(items[i]["y"]), oracle.bitlinear(x, nw, packed, N, EPS)) <= 1e-3


def test_batched_refused_during_capture():
    items = _mixed_items(28, [(40, 1024, 64, "plain")])
    bl.bitlinear_forward_batched(items)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        with pytest.raises(bl.BitLinearError) as e:
            bl.bitlinear_forward_batched(items)
    assert e.value.status == bl.BL_ERR_UNSUPPORTED


def test_captured_forward_survives_workspace_growth_and_release():
    # A graph captured around an unfused forward holds the workspace's
    # address.  A later, larger call on the same stream grows the workspace
    # and bl_release_workspace frees what it can: the captured buffer must
    # stay allocated, so replays keep reproducing the eager result.
    M, K, N = 40, 1024, 256
    x, nw, packed, scale = proj_inputs(29, 0, 0, M, K, N)
    dx, dn, dp = dev(x), dev(nw), dev(packed)
    s = torch.cuda.Stream()
    y = torch.full((M, N), float("nan"), device=DEV)
    with torch.cuda.stream(s):
        ref = bl.bitlinear_forward(dx, dn, dp, scale, N, EPS)  # workspace of s exists
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        bl.bitlinear_forward(dx, dn, dp, scale, N, EPS, y=y)
    M2, K2, N2 = 4096, 3072, 512
    x2, nw2, packed2, scale2 = proj_inputs(29, 1, 0, M2, K2, N2)
    with torch.cuda.stream(s):
        y2 = bl.bitlinear_forward(dev(x2), dev(nw2), dev(packed2), scale2, N2, EPS)
    torch.cuda.synchronize()
    rows = inputs.sample_rows(M2, 8, seed=29)
    assert rel_l2(host(y2)[rows], oracle.bitlinear(x2[rows], nw2, packed2, N2, EPS)) <= 1e-3
    bl.bl_release_workspace()
    junk = torch.full((16 << 20,), 7.0, device=DEV)  # reuse of freed memory would show
    for rep in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {rep}"
    del junk


# --------------------------------------------------- weights from a GGUF file ---

def test_forward_from_gguf_image():
    # A Qwen3-shaped q projection and its float16 per-projection norm stored in
    # a GGUF image (tests/gguf_file.py), located with bl_gguf_find_tensor and
    # uploaded as they stand: the forward equals the oracle on the same bytes,
    # and the float32 forward on the widened norm bit for bit.
    import gguf_file as gg
    K, N, M = 1024, 2048, 5
    packed, scale = oracle.i2s_pack(inputs.weight(32, 0, 0, N, K))
    nw = inputs.norm_weight(32, 0, 0, K).astype(np.float16)
    img = gg.write([("general.architecture", gg.STRING, "qwen3")],
                   [("blk.0.attn_q_norm_in.weight", gg.T_F16, [K], nw.tobytes()),
                    ("blk.0.attn_q.weight", gg.T_I2S, [K, N], packed.tobytes())])
    buf, w_scale, K2, N2 = bl.gguf_i2s_weight(img, "blk.0.attn_q.weight")
    assert (K2, N2) == (K, N) and w_scale == scale
    t = bl.gguf_find_tensor(img, "blk.0.attn_q_norm_in.weight")
    nw_dev = dev(img[t["offset"]:t["offset"] + t["nbytes"]].copy()).view(torch.float16)
    x = inputs.activations(32, 0, 1, M, K)
    y = bl.bitlinear_forward(dev(x), nw_dev, dev(buf.copy()), w_scale, N, EPS)
    nw32 = oracle.half_to_float(nw.view(np.uint16))
    assert rel_l2(host(y), oracle.bitlinear(x, nw32, packed, N, EPS)) <= 1e-3
    y32 = bl.bitlinear_forward(dev(x), dev(nw32), dev(packed), scale, N, EPS)
    assert torch.equal(y, y32)


# ------------------------------------------------------- seeded shape sweep ---

def _sweep_shapes(seed: int, count: int, max_work: float = 2.5e8):
    """count seeded (M, K, N): decode rows (M <= 16) and tiled rows, K any
    multiple of 128 up to 4096 (odd superblock counts and ragged K blocks of a
    split included), N up to 1300, cut down where M*K*N exceeds max_work so
    that the oracle finishes each case in well under a second."""
    g = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        M = int(g.integers(1, 17)) if g.random() < 0.4 else int(g.integers(17, 1100))
        K = 128 * int(g.integers(1, 33))
        N = min(int(g.integers(1, 1301)), max(1, int(max_work // (M * K))))
        out.append((M, K, N))
    return out


SWEEP = _sweep_shapes(4242, 40)


def test_random_shape_sweep():
    # Each shape on its own: the raw product bit-exact against the oracle on
    # random codes, the forward equal to the fp32 epilogue of the two hooks
    # and within 1e-3 of the oracle.  Then every shape in one stateless
    # batched call (merged decode, shared planning, K splits where the plan
    # makes them), bit-identical to the single calls.
    items, singles = [], []
    for i, (M, K, N) in enumerate(SWEEP):
        log(f"sweep case {i}: M={M} K={K} N={N}")
        x, nw, packed, scale = proj_inputs(43, i, 0, M, K, N)
        dx, dn, dp = dev(x), dev(nw), dev(packed)
        codes = inputs.rng(43, i, 1, 7).integers(-127, 128, size=(M, K)).astype(np.int8)
        acc = bl.bitlinear_matmul_i32(dev(codes), dp, N)
        assert np.array_equal(host(acc), oracle.matmul_i32(codes, packed, K, N)), (M, K, N)
        y = bl.bitlinear_forward(dx, dn, dp, scale, N, EPS)
        xq, f = bl.bitlinear_quant(dx, dn, EPS)
        assert torch.equal(y, _hooks_epilogue(bl.bitlinear_matmul_i32(xq, dp, N), f, scale)), (M, K, N)
        assert rel_l2(host(y), oracle.bitlinear(x, nw, packed, N, EPS)) <= 1e-3, (M, K, N)
        items.append(dict(x=dx, norm_w=dn, packed_w=dp, w_scale=scale, eps=EPS, N=N,
                          y=torch.full((M, N), float("nan"), device=DEV)))
        singles.append(y)
    bl.bitlinear_forward_batched(items)
    torch.cuda.synchronize()
    for (M, K, N), it, y in zip(SWEEP, items, singles):
        assert torch.equal(it["y"], y), (M, K, N)
    log(f"sweep: {len(SWEEP)} shapes, batched call bit-identical to single calls")


def test_prefill_group_many_generations():
    # A prefill launch with more tiles than fit on the GPU at once (here 735
    # tiles of mixed K, ragged M and N, against 512 resident workgroups): a
    # workgroup whose successor exists then also touches that tile's
    # activation rows before it stores.  The outputs must equal the single
    # calls (launches of at most 96 tiles, which fit at once) bit for bit over
    # two forwards into NaN-filled outputs, and the oracle on sampled rows.
    specs = [(1000, 3200, 3000), (700, 640, 2900), (1000, 128, 3072), (300, 4096, 1000),
             (1000, 2176, 2600), (129, 1152, 257), (1000, 1024, 3072), (513, 3072, 1024),
             (1000, 2048, 2048), (900, 384, 3000), (1000, 1152, 2816), (257, 640, 33)]
    tiles = sum(-(-M // 128) * -(-N // 256) for M, K, N in specs)
    assert tiles > 2 * 256
    items, refs = [], []
    for i, (M, K, N) in enumerate(specs):
        x, nw, packed, scale = proj_inputs(44, i, 0, M, K, N, heavy=(i % 3 == 1))
        it = dict(x=dev(x), norm_w=dev(nw), packed_w=dev(packed), w_scale=scale, eps=EPS, N=N,
                  y=torch.full((M, N), float("nan"), device=DEV))
        items.append(it)
        refs.append((x, nw, packed))
    singles = [bl.bitlinear_forward(it["x"], it["norm_w"], it["packed_w"], it["w_scale"], it["N"], EPS)
               for it in items]
    with bl.Group(items) as g:
        assert [d["kind"] for d in g.forward_launches()][-1] == "prefill"
        for rep in range(2):
            for it in items:
                it["y"].fill_(float("nan"))
            g.forward()
            torch.cuda.synchronize()
            for (M, K, N), it, ys in zip(specs, items, singles):
                assert torch.equal(it["y"], ys), (rep, M, K, N)
    log(f"prefill group of {len(specs)} problems, {tiles} tiles: identical to single calls")
    for i in (0, 3, 7, 11):
        (M, K, N), (x, nw, packed) = specs[i], refs[i]
        rows = inputs.sample_rows(M, 8, seed=44 + i)
        ref = oracle.bitlinear(np.ascontiguousarray(x[rows]), nw, packed, N, EPS)
        assert rel_l2(host(singles[i])[rows], ref) <= 1e-3, (M, K, N)
