"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds only random-number generation and the shapes of the
workloads.  It contains none of the method's arithmetic (no quantization, no
packing, no normalisation), so the oracle and the GPU path can both be fed
from it without sharing any computation.

Shapes follow the model table and per-layer tensor widths of
"BitNet Embeddings GGUF Conversion Implementation" (s1 "Background",
"Per-Layer Tensors", s4.5 "load_tensors"): the norm width of each projection
is its input width K, and weights are [N, K] (output x input).

Generator: numpy PCG64 seeded by ``SeedSequence([workload, layer, proj, role])``
with role 0 = weight, 1 = norm weight, 2 = activations, 3 = outlier channels.
All values are drawn directly as float32.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

ROLE_W, ROLE_NORM, ROLE_X, ROLE_OUTLIER = 0, 1, 2, 3

EPS = 1e-6  # rms_norm_eps of both model families

# (name, K, N) for the seven BitLinears of one layer.
QWEN3_06B = (
    ("q", 1024, 2048), ("k", 1024, 1024), ("v", 1024, 1024), ("o", 2048, 1024),
    ("gate", 1024, 3072), ("up", 1024, 3072), ("down", 3072, 1024),
)
GEMMA3_270M = (
    ("q", 640, 1024), ("k", 640, 256), ("v", 640, 256), ("o", 1024, 640),
    ("gate", 640, 2048), ("up", 640, 2048), ("down", 2048, 640),
)
QWEN3_LAYERS = 28


@dataclass(frozen=True)
class Workload:
    """One of the five synthetic workloads."""
    cid: int            # 1..5
    name: str
    M: int              # token rows per BitLinear
    layers: int         # distinct layers (each with its own weights)
    projs: tuple        # (name, K, N) per BitLinear of a layer
    heavy_tail: bool = False

    @property
    def bitlinears(self) -> int:
        return self.layers * len(self.projs)


WORKLOADS = {
    1: Workload(1, "single BitLinear M=8 1024->3072", 8, 1, (("gate", 1024, 3072),)),
    2: Workload(2, "decode M=1 Qwen3-0.6B layer (7 BitLinears)", 1, 1, QWEN3_06B),
    3: Workload(3, "prefill M=512 Gemma3-270M layer (7 BitLinears)", 512, 1, GEMMA3_270M),
    4: Workload(4, "prefill M=16384 28-layer Qwen3-0.6B stack (196 BitLinears)", 16384,
                QWEN3_LAYERS, QWEN3_06B),
    5: Workload(5, "long-context M=32768 Qwen3-0.6B gate/up/down, heavy-tailed x", 32768, 1,
                tuple(p for p in QWEN3_06B if p[0] in ("gate", "up", "down")), True),
}


def rng(workload: int, layer: int, proj: int, role: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload, layer, proj, role])))


def weight(workload: int, layer: int, proj: int, N: int, K: int, std: float = 0.02) -> np.ndarray:
    """Full-precision weight [N, K] ~ N(0, std^2), float32."""
    return (rng(workload, layer, proj, ROLE_W).standard_normal((N, K), dtype=np.float32)
            * np.float32(std))


def norm_weight(workload: int, layer: int, proj: int, K: int) -> np.ndarray:
    """Per-projection norm weight [K] ~ N(1, 0.1^2), float32."""
    g = rng(workload, layer, proj, ROLE_NORM)
    return np.float32(1.0) + g.standard_normal(K, dtype=np.float32) * np.float32(0.1)


def activations(workload: int, layer: int, proj: int, M: int, K: int,
                heavy_tail: bool = False) -> np.ndarray:
    """Activations [M, K], float32.

    Normal: N(0, 1).  Heavy-tailed: Student-t with 3 degrees of freedom, then
    round(0.001*K) seeded channels (at least one) multiplied by 20 in every row.
    """
    g = rng(workload, layer, proj, ROLE_X)
    if not heavy_tail:
        return g.standard_normal((M, K), dtype=np.float32)
    x = g.standard_t(3, size=(M, K)).astype(np.float32)
    n_out = max(1, int(round(0.001 * K)))
    ch = rng(workload, layer, proj, ROLE_OUTLIER).choice(K, size=n_out, replace=False)
    x[:, ch] *= np.float32(20.0)
    return x


# Which projections of a layer read the same input: q, k and v normalise the
# attention input, gate and up the FFN input (each with its own norm weight);
# o and down have inputs of their own.  Value: the projection index whose
# seed stands for the shared input.
SHARED_INPUT = {"q": 0, "k": 0, "v": 0, "o": 3, "gate": 4, "up": 4, "down": 6}


def activations_device(torch, workload: int, layer: int, proj: int, M: int, K: int, device):
    """Activations [M, K] ~ N(0, 1), float32, drawn on `device` by torch's
    generator seeded from SeedSequence([workload, layer, proj, ROLE_X]).

    For inputs too large to draw on the host in reasonable time (a stream of
    numbers different from `activations`; nothing compares the two).
    """
    seed = int(np.random.SeedSequence([workload, layer, proj, ROLE_X]).generate_state(1, np.uint64)[0] >> 1)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((M, K), generator=g, device=device, dtype=torch.float32)


def sample_rows(M: int, count: int, seed: int = 0) -> np.ndarray:
    """Sorted distinct row indices, always including the first and the last."""
    if M <= count:
        return np.arange(M)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([0x5A, M, count, seed])))
    mid = g.choice(np.arange(1, M - 1), size=count - 2, replace=False)
    return np.sort(np.concatenate([[0, M - 1], mid]))


def tile_rows(M: int, tile: int, seed: int = 0) -> np.ndarray:
    """Sorted distinct row indices: one seeded row inside every block of
    `tile` consecutive rows (so every row tile of a tiled kernel is hit),
    plus the first and the last row."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([0x7A, M, tile, seed])))
    starts = np.arange(0, M, tile)
    picks = starts + (g.random(len(starts)) * np.minimum(tile, M - starts)).astype(np.int64)
    return np.unique(np.concatenate([[0, M - 1], picks]))
