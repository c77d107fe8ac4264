"""Writes tests/golden/fullsize_oracle.npz: float32 oracle outputs of the full
AuraFlow transformer (4 joint + 32 single blocks, d = 3072, seeded bf16 weights)
for the full-size GPU parity tests, so those tests need not rerun minutes of
CPU oracle work on every GPU run. Calls only the oracle and the seeded input
generators (through tests/helpers.py, which holds no model arithmetic).

Entries (each with an input checksum the tests recompute, so a change to the
input recipe is caught):
  d1536        bf16 forward at 1536^2 (latent 4x192x192, 9216 image tokens, the
               whole 96x96 PE grid), CFG batch 2, text 256 tokens with seeded
               valid lengths                                      [2, 4, 192, 192]
  c1024_mx     the same workload at 1024^2 in MXFP8 mode (oracle mx=True)
                                                                  [2, 4, 128, 128]
  c1024_mx_ulp the MXFP8 forward of the same inputs with every latent moved up
               by one float32 ulp: the oracle's own sensitivity, which bounds how
               closely any implementation that is not bit-identical can agree
                                                                  [2, 4, 128, 128]
  e1024_b8     samples 1 (uncond, image 1) and 6 (cond, image 2) of the batch-8
               CFG forward of the 4-image sampling workload at step 10 of 25
               (tau = sigma_10, shift 1.73)                       [2, 4, 128, 128]

    python tests/golden/make_fullsize_golden.py [--threads N] [--only NAME]
"""
from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import oracle  # noqa: E402
import seeded_inputs  # noqa: E402
from helpers import PrefetchWeights, workload_inputs  # noqa: E402

OUT = os.path.join(HERE, "fullsize_oracle.npz")
E_SAMPLES = (1, 6)


def full_cfg():
    return oracle.AuraFlowConfig(ln_eps=float(np.float32(1e-6)))


def cd_inputs(H, W):
    """The CFG batch-2 inputs of the full-size tests: one latent and one timestep
    shared by both halves, independent text rows, seeded valid lengths."""
    lengths = seeded_inputs.valid_lengths(2, 16, 256)
    lat, taus, text, mask = workload_inputs(2, 4, H, W, 256, 2048, lengths=lengths, cfg_pairs=True)
    return lat, taus, oracle.round_bf16(text), mask


def e_inputs():
    """Batch 8 = [4 uncond; 4 cond] of the 4-image sampling workload at step 10:
    latents x0 duplicated, every row at tau = sigma_10 (float32), text rows drawn
    independently (streams 100.. uncond, 200.. cond), seeded valid lengths."""
    Bp, T = 4, 256
    x0 = seeded_inputs.latents(Bp, 4, 128, 128, first_index=300)
    sig = oracle.sigma_schedule(25, 1.73)
    tau = np.full(2 * Bp, np.float32(sig[10]), np.float32)
    text = np.concatenate([seeded_inputs.text_embeddings(Bp, T, 2048, first_index=100),
                           seeded_inputs.text_embeddings(Bp, T, 2048, first_index=200)])
    lengths = np.concatenate([seeded_inputs.valid_lengths(Bp, 16, T, seed=5),
                              seeded_inputs.valid_lengths(Bp, 16, T, seed=6)])
    mask = seeded_inputs.length_mask(lengths, T)
    return np.concatenate([x0, x0]), tau, oracle.round_bf16(text), mask


def ulp_up(inputs):
    """The same inputs with every latent moved to the next float32 value above it."""
    lat, taus, text, mask = inputs
    return np.nextafter(lat, np.float32(np.inf)).astype(np.float32), taus, text, mask


def checksum(*arrays):
    return np.array([float(np.asarray(a, np.float64).sum()) for a in arrays], np.float64)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--threads", type=int, default=min(16, len(os.sched_getaffinity(0))))
    ap.add_argument("--only", default=None)
    a = ap.parse_args()
    cfg = full_cfg()
    out = dict(np.load(OUT)) if os.path.exists(OUT) else {}
    jobs = {
        "d1536": lambda: (cd_inputs(192, 192), False, None),
        "c1024_mx": lambda: (cd_inputs(128, 128), True, None),
        "c1024_mx_ulp": lambda: (ulp_up(cd_inputs(128, 128)), True, None),
        "e1024_b8": lambda: (e_inputs(), False, E_SAMPLES),
    }
    for name, job in jobs.items():
        if a.only and name != a.only:
            continue
        (lat, taus, text, mask), mx, rows = job()
        out[name + "_checksum"] = checksum(lat, taus, text, mask)
        if rows is not None:
            idx = list(rows)
            lat, taus, text, mask = lat[idx], taus[idx], text[idx], mask[idx]
        t0 = time.time()
        W = PrefetchWeights(cfg, threads=a.threads).as_weights()
        ref = oracle.forward(cfg, W, lat, taus, text, mask, np.float32, mx=mx)
        out[name] = ref.astype(np.float32)
        print(f"{name}: {ref.shape} in {time.time() - t0:.0f} s", flush=True)
        np.savez_compressed(OUT, **out)


if __name__ == "__main__":
    main()
