"""Entry noising, Residual CFG and the per-slot latent update.

StreamDiffusion paper notes, section 2 (R-CFG):
* virtual residual noise   eps' = (x_tau - sqrt(alpha_tau) x0*) / sqrt(beta_tau)
* combine                  eps_cfg = delta eps' + gamma (eps_c - delta eps')
* self-negative: x0* is the frame's own input latent (n forwards in total);
  onetime-negative: one negative forward (n+1 forwards in total).
* full CFG, the standard guidance R-CFG replaces (2n forwards): eps' is the
  denoiser's own prediction under the negative prompt for the same latent and
  timestep; with delta = 1 the combine is eps_u + gamma (eps_c - eps_u).

The pages name no sampler.  Reading: deterministic DDIM (eta = 0):
x0_hat = (x_tau - b_tau eps_cfg) / a_tau, the next slot receives
a_next x0_hat + b_next eps_cfg, the last slot emits x0_hat.  The LCM-style
variant (the pages pair the pipeline with LCM models) re-noises x0_hat with
fresh noise z instead: a_next x0_hat + b_next z, z drawn per frame and slot and
passed in with the frame.

Pins (tests/test_oracle_guidance.py): gamma = 1 gives eps_c; delta = 0 gives
gamma eps_c; at the entry slot the virtual residual equals the entry noise;
eps_cfg equal to the true noise recovers x0; the identity pipeline
(eps_c := eps') emits every input unchanged.
"""
from __future__ import annotations


def entry_noise(x0, eps, a, b):
    """x_tau0 = a x0 + b eps (the noising that starts a frame's trajectory)."""
    return a * x0 + b * eps


def virtual_residual(x_tau, x0_star, a, b):
    """eps' = (x_tau - a x0*) / b."""
    return (x_tau - a * x0_star) / b


def rcfg(eps_c, eps_p, gamma, delta):
    """eps_cfg = delta eps' + gamma (eps_c - delta eps')."""
    return delta * eps_p + gamma * (eps_c - delta * eps_p)


def predict_x0(x_tau, eps, a, b):
    return (x_tau - b * eps) / a


def renoise(x0_hat, eps, a_next, b_next):
    return a_next * x0_hat + b_next * eps
