"""Seeded synthetic inputs for the serial Markov draft walk.

This module serves both the oracle side and the GPU side and holds none of the
walk's arithmetic: it draws random numbers with numpy's PCG64 and casts them
to bf16 with torch's own float32 -> bfloat16 conversion.  bf16 tensors are
returned as ``uint16`` bit patterns.

Recipe (stand-ins for the trained drafter weights and the prompts the pages
measure with, which are not available):
  * weights, one generator per workload, seed = workload index:
      W1 = bf16(N(0, 1))      [V, r]
      W2 = bf16(0.02 * N(0, 1)) [V, r]   (0.02 is a standard deviation)
  * per round, seed = 1_000_000 * workload + round:
      base     = bf16(2 * N(0, 1))       [B, gamma, V]
      anchor   ~ U{0 .. V-1}             [B]
      T        from {0, 0.6, 1.0}        [B]   (or all 0 for greedy workloads)
      uniforms ~ U[0, 1) float32         [B, gamma]
  * int8 variant: one fp32 scale per row, scale = rowmax|w| / 127,
    q = clamp(round_half_even(w / scale), -127, 127); an all-zero row has
    scale 0 and q 0.  The harness quantises once and both sides read (q, scale).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

R = 256
TEMPS = (0.0, 0.6, 1.0)


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    V: int
    gamma: int
    batches: tuple
    temps: str            # "greedy" | "mixed" | "cycle"
    rounds: int
    w2_dtypes: tuple = ("bf16",)
    note: str = field(default="")


# The five workloads the walk is measured and checked on.
WORKLOADS = {
    0: Workload(0, "toy_v32000_g7", 32_000, 7, (1,), "greedy", 1000,
                note="toy Markov walk, greedy"),
    1: Workload(1, "qwen3_vocab_v151936_g7", 151_936, 7, (1,), "greedy", 1000,
                note="Qwen3-size vocabulary, greedy, 1000 seeded rounds"),
    2: Workload(2, "long_walk_v151936_g16", 151_936, 16, (1, 4, 16), "mixed", 200,
                note="gamma=16 with per-request temperature in {0, 0.6, 1.0}"),
    3: Workload(3, "large_vocab_v248320_g16", 248_320, 16, (1,), "greedy", 200,
                w2_dtypes=("bf16", "int8"),
                note="residency stress; bf16 and int8+row-scale W2"),
    4: Workload(4, "batched_v129280_g5", 129_280, 5, (64, 128, 253), "mixed", 100,
                note="batched walk, mixed temperatures"),
}


def to_bf16_bits(x) -> np.ndarray:
    """float32/float64 array -> bf16 bit patterns, via torch's round-to-nearest-even cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def weights(index: int, V: int | None = None, r: int = R, w2_std: float = 0.02):
    """(W1, W2) bf16 bit patterns [V, r] for workload ``index`` (seed = index)."""
    V = WORKLOADS[index].V if V is None else V
    rng = np.random.Generator(np.random.PCG64(index))
    W1 = to_bf16_bits(rng.standard_normal((V, r), dtype=np.float32))
    W2 = to_bf16_bits(w2_std * rng.standard_normal((V, r), dtype=np.float32))
    return W1, W2


def quantize_int8(W2_bits: np.ndarray):
    """One fp32 scale per row (rowmax|w| / 127) and int8 codes rounded half to even."""
    w = (np.ascontiguousarray(W2_bits, dtype=np.uint16).astype(np.uint32) << 16)
    w = w.view(np.float32).astype(np.float64)
    scale = (np.abs(w).max(axis=1) / 127.0).astype(np.float32)
    s = scale.astype(np.float64)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(w / np.where(s > 0, s, 1.0)), 0.0)
    q = np.clip(q, -127, 127).astype(np.int8)
    return q, scale


def temperatures(rng, B: int, mode: str, round_index: int) -> np.ndarray:
    if mode == "greedy":
        return np.zeros(B, dtype=np.float32)
    if mode == "cycle" or (mode == "mixed" and B == 1):
        return np.full(B, TEMPS[round_index % 3], dtype=np.float32)
    return np.asarray(TEMPS, dtype=np.float32)[rng.integers(0, 3, size=B)]


def round_inputs(index: int, round_index: int, B: int, gamma: int | None = None,
                 V: int | None = None, temps: str | None = None, base_std: float = 2.0):
    """Per-round tensors: base [B,gamma,V] u16, anchor [B] i32, T [B] f32, uniforms [B,gamma] f32."""
    wl = WORKLOADS[index]
    V = wl.V if V is None else V
    gamma = wl.gamma if gamma is None else gamma
    temps = wl.temps if temps is None else temps
    rng = np.random.Generator(np.random.PCG64(1_000_000 * index + round_index))
    base = to_bf16_bits(base_std * rng.standard_normal((B, gamma, V), dtype=np.float32))
    anchor = rng.integers(0, V, size=B).astype(np.int32)
    T = temperatures(rng, B, temps, round_index)
    uniforms = rng.random((B, gamma), dtype=np.float32)
    return {"base": base, "anchor": anchor, "T": T, "uniforms": uniforms}


def toy(seed: int, V: int = 12, r: int = 4, B: int = 1, gamma: int = 3, w2_std: float = 0.5,
        base_std: float = 1.0, temps: str = "greedy"):
    """Tiny walk for brute-force pins (the pages' Fig 2 size is V=12, r=4, three steps)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    W1 = to_bf16_bits(rng.standard_normal((V, r), dtype=np.float32))
    W2 = to_bf16_bits(w2_std * rng.standard_normal((V, r), dtype=np.float32))
    base = to_bf16_bits(base_std * rng.standard_normal((B, gamma, V), dtype=np.float32))
    anchor = rng.integers(0, V, size=B).astype(np.int32)
    T = temperatures(rng, B, temps, seed)
    uniforms = rng.random((B, gamma), dtype=np.float32)
    return {"W1": W1, "W2": W2, "base": base, "anchor": anchor, "T": T, "uniforms": uniforms}


def gru_cell_weights(index: int, r: int = R, gates: int = 3):
    """Synthetic cell for the recurrent serial heads (the pages measure such heads
    on synthetic weights): Wih, Whh [gates * r, r] bf16 bits and bih, bhh
    [gates * r] f32, all N(0, 1/r), the scale of the usual
    uniform(-1/sqrt(r), 1/sqrt(r)) init.  gates = 3: the GRU, 1: the RNN."""
    rng = np.random.Generator(np.random.PCG64(7_000 + 10 * index + gates))
    sd = 1.0 / np.sqrt(r)
    Wih = to_bf16_bits(sd * rng.standard_normal((gates * r, r), dtype=np.float32))
    Whh = to_bf16_bits(sd * rng.standard_normal((gates * r, r), dtype=np.float32))
    bih = (sd * rng.standard_normal(gates * r)).astype(np.float32)
    bhh = (sd * rng.standard_normal(gates * r)).astype(np.float32)
    return Wih, Whh, bih, bhh


def rnn_cell_weights(index: int, r: int = R):
    """Synthetic tanh RNN cell: Wih, Whh [r, r] bf16 bits, bih, bhh [r] f32."""
    return gru_cell_weights(index, r=r, gates=1)


def gated_weights(index: int, r: int = R):
    """Synthetic gated head: the r x r gate matrix drawn N(0, 1/r), quantised
    like int8 W2 rows (Gq [r, r] int8 codes, gs [r] f32 row scales), and a gate
    bias gb [r] f32 drawn N(0, 1), so that the gates spread over (0, 1)."""
    rng = np.random.Generator(np.random.PCG64(7_500 + index))
    G = to_bf16_bits((1.0 / np.sqrt(r)) * rng.standard_normal((r, r), dtype=np.float32))
    Gq, gs = quantize_int8(G)
    gb = rng.standard_normal(r).astype(np.float32)
    return Gq, gs, gb


DOMINO_D = 2560  # the drafter's hidden width (the Qwen3-4B target the pages' Domino runs use)


def domino_cell_weights(index: int, d: int = DOMINO_D, r: int = R):
    """Synthetic Domino cell: a GRU whose input is [W1[prev]; H_k], Wih [3r, r + d]
    bf16 bits drawn N(0, 1/(r + d)) so that the wide input keeps the gates in
    range, Whh [3r, r] bf16 bits and both biases N(0, 1/r)."""
    rng = np.random.Generator(np.random.PCG64(7_700 + index))
    Wih = to_bf16_bits((1.0 / np.sqrt(r + d)) * rng.standard_normal((3 * r, r + d), dtype=np.float32))
    sd = 1.0 / np.sqrt(r)
    Whh = to_bf16_bits(sd * rng.standard_normal((3 * r, r), dtype=np.float32))
    bih = (sd * rng.standard_normal(3 * r)).astype(np.float32)
    bhh = (sd * rng.standard_normal(3 * r)).astype(np.float32)
    return Wih, Whh, bih, bhh


def domino_hidden(index: int, round_index: int, B: int, gamma: int, d: int = DOMINO_D):
    """The drafter's hidden states of one round, [B, gamma, d] bf16 bits, N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(9_000_000 + 1000 * index + round_index))
    return to_bf16_bits(rng.standard_normal((B, gamma, d), dtype=np.float32))


def gru_h0(index: int, round_index: int, B: int, r: int = R):
    """Initial GRU states [B, r] f32 in (-1, 1): tanh of N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(8_000_000 + 1000 * index + round_index))
    return np.tanh(rng.standard_normal((B, r))).astype(np.float32)
