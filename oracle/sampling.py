"""Flow-matching schedule and the Euler + classifier-free-guidance update (TEST INFRASTRUCTURE ONLY).

[PIPE] AuraFlowPipeline 核心参数详解: guidance is off for guidance_scale <= 1; the
denoising loop combines noise_pred_uncond + s * (noise_pred_text - noise_pred_uncond).
[TRANS] 在 AuraFlowPipeline 中的实际调用: latents are duplicated for CFG, the output is
split with chunk(2) as (uncond, text), t = 1 is noise and t = 0 the image.
[DEEP] 2.3 (流匹配调度器): 1000 train timesteps, shift 1.73.
"""
from __future__ import annotations

import numpy as np


def sigma_schedule(num_steps: int, shift: float = 1.73) -> np.ndarray:
    """sigma_0..sigma_N (float64): u_i = 1 - i/N mapped through s*u / (1 + (s-1)*u).

    The pages give only the shift and the train-timestep count; the uniform grid
    in u followed by the timestep-shift map is the reading taken (sigma_0 = 1,
    sigma_N = 0, monotone decreasing). The transformer receives tau_i = sigma_i.
    """
    i = np.arange(num_steps + 1, dtype=np.float64)
    u = 1.0 - i / num_steps
    return shift * u / (1.0 + (shift - 1.0) * u)


def cfg_combine(v, guidance: float):
    """v = [uncond (B'); cond (B')] -> uncond + s (cond - uncond) when s > 1, else v unchanged."""
    if guidance <= 1.0:
        return v
    half = v.shape[0] // 2
    vu, vc = v[:half], v[half:]
    return vu + guidance * (vc - vu)


def euler_step(x, v_hat, sigma: float, sigma_next: float):
    """x + (sigma_next - sigma) * v_hat."""
    return x + (sigma_next - sigma) * v_hat


def cfg_euler_step(x, v, sigma: float, sigma_next: float, guidance: float):
    return euler_step(x, cfg_combine(v, guidance), sigma, sigma_next)
