"""The sampler around the stack: eight steps over the pages' timesteps (test infrastructure only).

[TRIM] "Trim 改变了什么", training bullet: the model is trained for eight-step DMD2 sampling at the
timesteps 999, 874, 749, 624, 500, 375, 250 and 125.  [TRIM] "在 ComfyUI 中运行": the template runs
8 steps of res_multistep with the simple schedule, and a sigma-shift node set to 10 on video and 3 on
audio.

Readings (the pages name the sampler; they do not write it out):
* noise level: sigma = t / 1000 for the listed t, and the rectified-flow parametrization
  x_sigma = (1 - sigma) x0 + sigma eps (alpha = 1 - sigma), sigma = 0 the clean latent;
* sigma shift s: sigma' = s sigma / (1 + (s - 1) sigma) (the time shift of rectified-flow
  transformers, Esser et al. 2024), s = 10 on the video tokens and 3 on the audio tokens, so the two
  modalities follow two schedules through the same eight steps; a final sigma' = 0 ends both;
* the stack's output stands for the velocity v = eps - x0 of the tokens it was given (the model's
  latent head -- final norm, projection to latent channels, unpatchify -- is not on the pages and is
  taken as the identity, so the latent is the token sequence itself); the denoised estimate is
  x0_hat = x - sigma' v;
* the start: x = sigma'_0 eps (an empty latent noised to the first level);
* res_multistep: a two-step exponential integrator in the data prediction (the multistep form of the
  refined exponential solver, Zhang, Tao & Chen 2023, "Improved order analysis and design of
  exponential integrator for diffusion models").  With lambda = log(alpha / sigma) the probability-flow
  ODE reads d(x / sigma)/d lambda = e^lambda x0_hat; taking x0_hat linear in lambda through the
  current and previous estimates and integrating exactly over a step of length h gives
      x_next = (sigma_next / sigma) x + alpha_next [(1 - e^-h) D0 + (h - 1 + e^-h) / h_prev D1],
      D0 = x0_hat_i,  D1 = x0_hat_i - x0_hat_{i-1},  h = lambda_next - lambda_i,
  first order (D1 = 0) at the first step, which has no previous estimate, and at the last step,
  whose target sigma = 0 has lambda = infinity (the step then returns x0_hat).
Everything is float64.
"""
from __future__ import annotations

import math

import numpy as np

N_STEPS = 8
SHIFT_VIDEO = 10.0
SHIFT_AUDIO = 3.0


def timesteps(n: int = N_STEPS) -> np.ndarray:
    """The n sampler timesteps: rint of n evenly spaced points from 999 down to (not including) 0
    (ties to even).  For n = 8 these are the pages' 999, 874, 749, 624, 500, 375, 250, 125."""
    return np.rint(np.linspace(999.0, 0.0, n + 1)[:n])


def shift(sigma, s: float):
    """Time shift sigma' = s sigma / (1 + (s - 1) sigma)."""
    sigma = np.asarray(sigma, dtype=np.float64)
    return s * sigma / (1.0 + (s - 1.0) * sigma)


def sigmas(s: float, ts=None) -> np.ndarray:
    """The n + 1 noise levels of one modality: shift(t / 1000) for the sampler timesteps, then 0."""
    ts = timesteps() if ts is None else np.asarray(ts, dtype=np.float64)
    return np.concatenate([shift(ts / 1000.0, s), [0.0]])


def lam(sigma: float) -> float:
    """lambda = log(alpha / sigma), alpha = 1 - sigma (+infinity at sigma = 0)."""
    return math.inf if sigma == 0.0 else math.log((1.0 - sigma) / sigma)


def step_coefficients(sig: np.ndarray, i: int) -> tuple[float, float, float, float]:
    """(sigma_i, a, b, c) of step i: x0_hat = x - sigma_i v; x_next = a x + b x0_hat_i + c x0_hat_{i-1}."""
    s0, s1 = float(sig[i]), float(sig[i + 1])
    if s1 == 0.0:
        return s0, 0.0, 1.0, 0.0                     # to the clean latent: x_next = x0_hat
    h = lam(s1) - lam(s0)
    alpha1 = 1.0 - s1
    a = s1 / s0
    b = alpha1 * (1.0 - math.exp(-h))                # = alpha1 - alpha0 sigma1 / sigma0, exactly
    c = 0.0
    if i > 0:
        h_prev = lam(s0) - lam(float(sig[i - 1]))
        k = alpha1 * (h - 1.0 + math.exp(-h)) / h_prev
        b, c = b + k, -k
    return s0, a, b, c


def step(x, v, x0_prev, sig: np.ndarray, i: int):
    """One sampler step on float64 arrays: returns (x_next, x0_hat_i)."""
    s0, a, b, c = step_coefficients(sig, i)
    x = np.asarray(x, dtype=np.float64)
    x0_hat = x - s0 * np.asarray(v, dtype=np.float64)
    x_next = a * x + b * x0_hat
    if c != 0.0:
        x_next = x_next + c * np.asarray(x0_prev, dtype=np.float64)
    return x_next, x0_hat


def start(eps, sig0: float):
    """The first state: sigma'_0 eps."""
    return sig0 * np.asarray(eps, dtype=np.float64)


def sample(eps, model, L_video: int, ts=None, s_video: float = SHIFT_VIDEO, s_audio: float = SHIFT_AUDIO,
           keep: bool = False):
    """The whole loop on [L][d] float64 tokens (rows < L_video video, the rest audio).  model(x, i, t)
    returns the velocity for state x at step i (timestep t).  Returns the final latent (and, with
    keep, the list of states and velocities)."""
    ts = timesteps() if ts is None else np.asarray(ts, dtype=np.float64)
    sv, sa = sigmas(s_video, ts), sigmas(s_audio, ts)
    x = np.empty_like(np.asarray(eps, dtype=np.float64))
    x[:L_video] = start(eps[:L_video], sv[0])
    x[L_video:] = start(eps[L_video:], sa[0])
    x0p = np.zeros_like(x)
    states, vels = [x.copy()], []
    for i, t in enumerate(ts):
        v = np.asarray(model(x, i, float(t)), dtype=np.float64)
        vels.append(v)
        xn, x0h = np.empty_like(x), np.empty_like(x)
        xn[:L_video], x0h[:L_video] = step(x[:L_video], v[:L_video], x0p[:L_video], sv, i)
        xn[L_video:], x0h[L_video:] = step(x[L_video:], v[L_video:], x0p[L_video:], sa, i)
        x, x0p = xn, x0h
        states.append(x.copy())
    return (x, states, vels) if keep else x
