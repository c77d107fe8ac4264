"""Writes tests/golden/vae_oracle.npz: float32 crops of the oracle's VAE decode of one
1024 x 1024 image (latent 4 x 128 x 128, seeded weights rounded to bf16), for the
full-size GPU parity test, so that test need not rerun minutes of CPU oracle work.
Calls only the oracle and the seeded generators.

Entries:
  full1024_center   image[0, :, 384:640, 384:640]        [3, 256, 256]
  full1024_corners  the four 64 x 64 corners (zero-padding edges), stacked
                    top-left, top-right, bottom-left, bottom-right      [4, 3, 64, 64]
  full1024_mean     per-channel mean of the whole image                 [3]
  full1024_checksum sum of the input latent (recomputed by the test)

    python tests/golden/make_vae_golden.py [--threads N]
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

OUT = os.path.join(HERE, "vae_oracle.npz")
LATENT_INDEX = 300      # the first latent of the 4-image sampling workload


def latent():
    import seeded_inputs
    return seeded_inputs.latents(1, 4, 128, 128, first_index=LATENT_INDEX)


def crops(img):
    c = img[0, :, 384:640, 384:640]
    k = np.stack([img[0, :, :64, :64], img[0, :, :64, -64:], img[0, :, -64:, :64], img[0, :, -64:, -64:]])
    return np.ascontiguousarray(c), np.ascontiguousarray(k), img[0].mean(axis=(1, 2))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--threads", type=int, default=None)
    ap.parse_args()
    import seeded_inputs
    from oracle import vae as V
    cfg = V.VAE_FULL
    W = V.VAEWeights.seeded(cfg, seeded_inputs.SEED_VAE_WEIGHTS, bf16=True)
    lat = latent()
    t0 = time.time()
    img = V.decode(cfg, W, lat, np.float32)
    c, k, m = crops(img)
    np.savez_compressed(OUT, full1024_center=c.astype(np.float32), full1024_corners=k.astype(np.float32),
                        full1024_mean=m.astype(np.float64), full1024_checksum=np.float64(lat.astype(np.float64).sum()))
    print(f"full1024: {img.shape} in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main()
