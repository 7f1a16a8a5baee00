"""Seeded synthetic inputs for the weight-only quantized product.

This module only draws random numbers and stores them in the storage types the
method consumes (int8 codes, IEEE binary16 scale bit patterns, OCP E4M3 bytes,
float32 row scales, bfloat16 activation bit patterns).  It contains none of the
method's arithmetic, so both the CPU oracle (tests) and the GPU library (tests,
benchmark) can take their inputs from here without sharing any computation.

Workload shapes follow the Qwen3.8-27B dimensions given on the NInfer model
cards (jabbatheduck/ninfer-ext-models, "Qwen3.8-27B EXL3" -> "Model": hidden
5120, intermediate 17408, vocabulary 248,320).  Value distributions are the
ones the benchmark definition fixes: uniform codes over the full two's
complement range, |N(0,1)|*c scales with a random sign, bf16 N(0,1) activations,
FP8 bytes uniform over the 254 finite encodings.

Draw order for every workload: codes, scale magnitudes, scale signs, activations.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np
import torch

Q4, Q5, Q6, FP8 = 4, 5, 6, 8
Q8 = 9          # groupwise 8-bit codes (the format id is not the bit width: 8 is FP8)
GROUP = 64


def code_bits(fmt: int) -> int:
    """Bits per code of a groupwise format id (4, 5, 6 or Q8 -> 8); 0 for FP8."""
    return {Q4: 4, Q5: 5, Q6: 6, Q8: 8}.get(fmt, 0)


@dataclasses.dataclass
class Workload:
    """One synthetic matrix plus activations.

    fmt      4/5/6 (and Q8 = 9) for groupwise codes, 8 for row-scaled FP8 E4M3.
    codes    int8 [M, K] two's complement codes (groupwise) or uint8 [M, K] E4M3 bytes (FP8).
    scales   uint16 [M, K/64] binary16 bit patterns (groupwise) or float32 [M] (FP8).
    x        uint16 [T, K] bfloat16 bit patterns.
    """
    name: str
    fmt: int
    M: int
    K: int
    T: int
    codes: np.ndarray
    scales: np.ndarray
    x: np.ndarray

    @property
    def weight_bytes(self) -> int:
        """Bytes of stored weight information per the format definition (codes + scales)."""
        if self.fmt == FP8:
            return self.M * self.K + 4 * self.M
        return self.M * self.K * code_bits(self.fmt) // 8 + 2 * self.M * (self.K // GROUP)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def draw_group_codes(gen: torch.Generator, bits: int, M: int, K: int) -> np.ndarray:
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1))
    return torch.randint(lo, hi, (M, K), generator=gen, dtype=torch.int8).numpy()


def draw_group_scales(gen: torch.Generator, M: int, G: int, mult: float) -> np.ndarray:
    mag = torch.randn((M, G), generator=gen, dtype=torch.float32).abs_() * mult
    sign = torch.randint(0, 2, (M, G), generator=gen, dtype=torch.int8).to(torch.float32) * 2 - 1
    return (mag * sign).to(torch.float16).view(torch.int16).numpy().view(np.uint16)


def draw_fp8_bytes(gen: torch.Generator, M: int, K: int) -> np.ndarray:
    # index 0..253 over the finite encodings, skipping 0x7F and 0xFF (the two NaNs)
    idx = torch.randint(0, 254, (M, K), generator=gen, dtype=torch.int16)
    idx += (idx >= 127).to(torch.int16)
    return idx.to(torch.uint8).numpy()


def draw_row_scales(gen: torch.Generator, M: int, mult: float) -> np.ndarray:
    return (torch.randn((M,), generator=gen, dtype=torch.float32).abs_() * mult).numpy()


def draw_activations(gen: torch.Generator, T: int, K: int) -> np.ndarray:
    x = torch.randn((T, K), generator=gen, dtype=torch.float32).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16)


def groupwise(name: str, fmt: int, M: int, K: int, T: int, scale_mult: float, seed: int = 0) -> Workload:
    """fmt: Q4, Q5, Q6 or Q8."""
    if K % GROUP:
        raise ValueError("K must be a multiple of 64")
    bits = code_bits(fmt)
    if not bits:
        raise ValueError(f"not a groupwise format: {fmt}")
    g = _gen(seed)
    codes = draw_group_codes(g, bits, M, K)
    scales = draw_group_scales(g, M, K // GROUP, scale_mult)
    x = draw_activations(g, T, K)
    return Workload(name, fmt, M, K, T, codes, scales, x)


def fp8_rows(name: str, M: int, K: int, T: int, scale_mult: float = 0.01, seed: int = 0) -> Workload:
    g = _gen(seed)
    codes = draw_fp8_bytes(g, M, K)
    # FP8 has no sign draw for the scale: one magnitude per row.
    scales = draw_row_scales(g, M, scale_mult)
    x = draw_activations(g, T, K)
    return Workload(name, FP8, M, K, T, codes, scales, x)


# The benchmark's named shapes.  Each entry: (fmt, M, K, list of T, scale multiplier).
CONFIGS: Dict[str, tuple] = {
    "q4_small_256x1024": (Q4, 256, 1024, [1], 0.01),
    "q4_gate_up_34816x5120": (Q4, 34816, 5120, [1, 4, 8], 0.01),
    "q5_down_5120x17408": (Q5, 5120, 17408, [1, 4], 0.01),
    "q6_head_248320x5120": (Q6, 248320, 5120, [1, 8], 0.005),
    "fp8_head_248320x5120": (FP8, 248320, 5120, [1, 8, 16], 0.01),
    "fp8_proj_5120x5120": (FP8, 5120, 5120, [1, 8, 16], 0.01),
    # the upstream artifact's 8-bit output head (the pages time its 8-token verify)
    "q8_head_248320x5120": (Q8, 248320, 5120, [1, 8], 0.0005),
    # the 131,072-row proposal head kept in the upstream 8-bit encoding, whose rows stand for
    # vocabulary ids through an index map
    "q8_proposal_head_131072x5120": (Q8, 131072, 5120, [1, 8, 16], 0.0005),
    # one GPU's share of an 8-way split: the Q6 head cut into row slices (248320 / 8 rows each)
    # and the Q5 down projection cut along K (17408 / 8 inputs each, partial sums added after)
    "q6_head_shard_31040x5120": (Q6, 31040, 5120, [1, 8], 0.005),
    "q5_down_kshard_5120x2176": (Q5, 5120, 2176, [1, 4], 0.01),
}


def config(name: str, T: Optional[int] = None, seed: int = 0) -> Workload:
    """Workload of a named shape; T defaults to the largest listed T (x rows 0..T-1 are
    the same draws whatever T is asked for only if T equals that maximum)."""
    fmt, M, K, Ts, mult = CONFIGS[name]
    T = max(Ts) if T is None else T
    if fmt == FP8:
        return fp8_rows(name, M, K, T, mult, seed)
    return groupwise(name, fmt, M, K, T, mult, seed)


def config_names() -> List[str]:
    return list(CONFIGS)


def logits(T: int, M: int, seed: int = 0, ties: bool = True) -> np.ndarray:
    """Synthetic output-head logits, float32 [T, M]: N(0, 1) * 3 with a few large values
    (draws: the values, then the positions and sizes of the large values); with ties, every
    token also gets groups of exactly equal values among its largest (copies of its own
    maximum and of other drawn values at random rows)."""
    g = _gen(seed)
    y = torch.randn((T, M), generator=g, dtype=torch.float32) * 3.0
    nbig = max(1, M // 4096)
    pos = torch.randint(0, M, (T, nbig), generator=g)
    big = torch.rand((T, nbig), generator=g) * 12.0 + 8.0
    y.scatter_(1, pos, big)
    if ties:
        npick = min(M, 8)
        src = torch.randint(0, M, (T, npick), generator=g)
        dst = torch.randint(0, M, (T, npick), generator=g)
        vals = torch.gather(y, 1, src)
        y.scatter_(1, dst, vals)
        top = y.max(dim=1, keepdim=True).values
        dst2 = torch.randint(0, M, (T, 2), generator=g)
        y.scatter_(1, dst2, top.expand(T, 2))
    return y.numpy()
