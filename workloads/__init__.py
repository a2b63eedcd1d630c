"""Seeded synthetic inputs for the Q4 group-32 quantized linear path.

This module only draws random numbers and lays out shapes. It holds none of the
method's arithmetic (no quantizer, no product) and is the one thing the CPU
oracle side and the HIP side both use: tests and the benchmark draw inputs here
and hand the same arrays to each.

Shapes follow the pages' model description (blog translation, pipeline
diagram; ONNX bundle README, usage section): the temporal transformer has 32
layers of width 4096 (32 heads x 128) with a gated FFN of width 11264; the
Depformer has 6 layers of width 1024 with a gated FFN of width 2816 and one
weight block per codebook step for 16 steps.

Recipe (stated once, used everywhere):
* generator: ``numpy.random.default_rng(SeedSequence([seed, config, layer, item, role]))``
  with role 0 for weights and 1 for activations;
* weights: ``standard_normal(dtype=float32) * float32(0.02)`` (std 0.02), fp32;
* activations: ``standard_normal(dtype=float32)`` (std 1), rounded to bf16
  (nearest, ties to even) and returned as uint16 bit patterns.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np

WEIGHT_STD = np.float32(0.02)
ROLE_WEIGHT = 0
ROLE_ACT = 1

# Temporal transformer (one layer): name, out (N), in (K), input stage.
HIDDEN = 4096
FFN = 11264
TEMPORAL_LAYERS = 32
# Stage ids name which activation vector feeds a linear: the attention input
# feeds q, k, v; the attention output feeds o; the FFN input feeds gate and up;
# the gated product feeds down.
STAGE_ATTN_IN, STAGE_ATTN_OUT, STAGE_FFN_IN, STAGE_FFN_MID = 0, 1, 2, 3
TEMPORAL_LINEARS: Tuple[Tuple[str, int, int, int], ...] = (
    ("q", HIDDEN, HIDDEN, STAGE_ATTN_IN),
    ("k", HIDDEN, HIDDEN, STAGE_ATTN_IN),
    ("v", HIDDEN, HIDDEN, STAGE_ATTN_IN),
    ("o", HIDDEN, HIDDEN, STAGE_ATTN_OUT),
    ("gate", FFN, HIDDEN, STAGE_FFN_IN),
    ("up", FFN, HIDDEN, STAGE_FFN_IN),
    ("down", HIDDEN, FFN, STAGE_FFN_MID),
)

# Depformer (one layer): each linear stored as [NUM_STEPS * out, in].
DEP_DIM = 1024
DEP_FFN = 2816
DEP_LAYERS = 6
DEP_STEPS = 16
DEPFORMER_LINEARS: Tuple[Tuple[str, int, int, int], ...] = (
    ("q", DEP_DIM, DEP_DIM, STAGE_ATTN_IN),
    ("k", DEP_DIM, DEP_DIM, STAGE_ATTN_IN),
    ("v", DEP_DIM, DEP_DIM, STAGE_ATTN_IN),
    ("o", DEP_DIM, DEP_DIM, STAGE_ATTN_OUT),
    ("gate", DEP_FFN, DEP_DIM, STAGE_FFN_IN),
    ("up", DEP_FFN, DEP_DIM, STAGE_FFN_IN),
    ("down", DEP_DIM, DEP_FFN, STAGE_FFN_MID),
)

# Token streams of one frame (blog translation, pipeline figure: 17 streams,
# text + 8 user audio + 8 assistant audio codebooks, summed into the step's
# input). Table sizes: the text table follows the 32k SentencePiece tokenizer
# of the ONNX bundle's file list; the pages give no audio codebook size, and
# 2048 entries (an 11-bit code) is the reading taken.
TEXT_VOCAB = 32000
AUDIO_CODEBOOK = 2048
TOKEN_STREAMS = 17

# Workload ids (1-based, in the order the benchmark configurations are listed).
CFG_GEMV, CFG_LAYER, CFG_STEP, CFG_DEPFORMER, CFG_SMALL_GEMM = 1, 2, 3, 4, 5


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


def rng(seed: int, config: int, layer: int, item: int, role: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, config, layer, item, role]))


def bf16_bits_rne(a: np.ndarray) -> np.ndarray:
    """Round fp32 samples to bf16 (nearest even) and return the bit patterns.

    Used only to produce bf16 activation inputs."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def weights(seed: int, config: int, layer: int, item: int, n: int, k: int) -> np.ndarray:
    """fp32 [n, k] weights, N(0, 0.02^2)."""
    g = rng(seed, config, layer, item, ROLE_WEIGHT)
    w = g.standard_normal((n, k), dtype=np.float32)
    w *= WEIGHT_STD
    return w


def activations(seed: int, config: int, layer: int, item: int, m: int, k: int) -> np.ndarray:
    """bf16 bit patterns [m, k], N(0, 1) rounded to bf16."""
    g = rng(seed, config, layer, item, ROLE_ACT)
    return bf16_bits_rne(g.standard_normal((m, k), dtype=np.float32))


def weights_many(specs: Sequence[Tuple[int, int, int, int, int, int]]) -> List[np.ndarray]:
    """Draw several weight matrices in parallel host threads (numpy releases the
    GIL while filling). specs: (seed, config, layer, item, n, k)."""
    with _cf.ThreadPoolExecutor(_threads()) as ex:
        return list(ex.map(lambda s: weights(*s), specs))


@dataclass(frozen=True)
class Linear:
    name: str
    n: int          # output features (rows of W)
    k: int          # input features
    stage: int      # which activation feeds it
    item: int       # index used in the seed


def temporal_layer() -> List[Linear]:
    return [Linear(nm, n, k, st, i) for i, (nm, n, k, st) in enumerate(TEMPORAL_LINEARS)]


def depformer_layer() -> List[Linear]:
    return [Linear(nm, n, k, st, i) for i, (nm, n, k, st) in enumerate(DEPFORMER_LINEARS)]


def weights_per_step() -> int:
    """Weights streamed by one 32-layer temporal step."""
    return TEMPORAL_LAYERS * sum(n * k for _, n, k, _ in TEMPORAL_LINEARS)


def depformer_weights_per_codebook_step() -> int:
    return DEP_LAYERS * sum(n * k for _, n, k, _ in DEPFORMER_LINEARS)

