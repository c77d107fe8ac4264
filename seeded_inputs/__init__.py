"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This module draws random numbers and nothing else: it holds none of the
transformer's arithmetic (no shapes derived from the model, no rounding, no
layout). Callers pass the shape and scale they want; both sides of a parity
test ask for the same (seed, index, shape, std) and get bit-identical float32
arrays.

Every stream is numpy's PCG64 seeded with ``SeedSequence([seed, index])`` so a
tensor can be regenerated on its own (the oracle streams weights block by block
without holding the whole model).

Seed roles used by the tests and the bench:
    0 weights (index = position in the canonical weight list)
    1 latents (index = sample)
    2 text embeddings (index = sample)
    3 valid text lengths (index = sample)
    4 timesteps (index = sample)
    5 text-encoder weights (index = position in the encoder's weight list)
    6 token ids (index = sample)
"""
from __future__ import annotations

import numpy as np

SEED_WEIGHTS = 0
SEED_LATENTS = 1
SEED_TEXT = 2
SEED_LENGTHS = 3
SEED_TIMESTEPS = 4
SEED_ENCODER_WEIGHTS = 5
SEED_TOKENS = 6
SEED_VAE_WEIGHTS = 7


def _gen(seed: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(index)])))


def normal(seed: int, index: int, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """float32 array of N(mean, std^2) draws for stream (seed, index)."""
    g = _gen(seed, index)
    a = g.standard_normal(size=tuple(int(s) for s in shape), dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return a


def uniform_int(seed: int, index: int, low: int, high_inclusive: int) -> int:
    """One integer drawn uniformly from [low, high_inclusive] for stream (seed, index)."""
    g = _gen(seed, index)
    return int(g.integers(low, high_inclusive + 1))


def uniform(seed: int, index: int, low: float, high: float) -> float:
    """One float64 drawn uniformly from [low, high) for stream (seed, index)."""
    g = _gen(seed, index)
    return float(g.uniform(low, high))


def latents(batch: int, channels: int, height: int, width: int, seed: int = SEED_LATENTS,
            first_index: int = 0) -> np.ndarray:
    """[batch, channels, height, width] float32 N(0,1); sample b uses stream first_index+b."""
    out = np.empty((batch, channels, height, width), np.float32)
    for b in range(batch):
        out[b] = normal(seed, first_index + b, (channels, height, width))
    return out


def text_embeddings(batch: int, tokens: int, dim: int, seed: int = SEED_TEXT,
                    first_index: int = 0) -> np.ndarray:
    """[batch, tokens, dim] float32 N(0,1); sample b uses stream first_index+b."""
    out = np.empty((batch, tokens, dim), np.float32)
    for b in range(batch):
        out[b] = normal(seed, first_index + b, (tokens, dim))
    return out


def valid_lengths(batch: int, low: int, high_inclusive: int, seed: int = SEED_LENGTHS) -> np.ndarray:
    """[batch] int64 lengths, each uniform in [low, high_inclusive]."""
    return np.array([uniform_int(seed, b, low, high_inclusive) for b in range(batch)], np.int64)


def length_mask(lengths: np.ndarray, tokens: int) -> np.ndarray:
    """[batch, tokens] uint8 with mask[b, j] = 1 iff j < lengths[b]."""
    j = np.arange(tokens)[None, :]
    return (j < np.asarray(lengths)[:, None]).astype(np.uint8)


def timesteps_uniform(batch: int, low: float = 0.0, high: float = 1000.0,
                      seed: int = SEED_TIMESTEPS) -> np.ndarray:
    """[batch] float64 timesteps t, uniform in [low, high)."""
    return np.array([uniform(seed, b, low, high) for b in range(batch)], np.float64)


def token_ids(batch: int, tokens: int, vocab: int, seed: int = SEED_TOKENS) -> np.ndarray:
    """[batch, tokens] int32 ids, each uniform in [0, vocab); sample b uses stream b."""
    out = np.empty((batch, tokens), np.int32)
    for b in range(batch):
        out[b] = _gen(seed, b).integers(0, vocab, size=tokens)
    return out
