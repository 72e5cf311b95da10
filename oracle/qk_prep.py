"""qk-RMSNorm and rotary position embedding before the cache write, in fp64.

What the step does (project page, "3.2 Fast Causal H3 VAE", iteration 6: after the qkv
projection, qk-norm, the rotary embedding and the K/V cache write run as one fused kernel;
iteration 3, inference item 2: the rotary position of a latent frame is applied a single
time, as the frame is written into its ring slot; iteration 4: frame tokens take the absolute
latent-frame index of the stream, so that every attention score depends only on time
differences).

The pages fix the order (normalise, rotate, write) and that positions are stream-absolute;
they do not print the formulas' details, so this module takes the plainest reading (listed
with the design notes):

  rms_norm   y_d = x_d / sqrt(mean_e x_e^2 + eps) * gamma_d      over head_dim, per head
  rope       head_dim is D/2 rotation pairs (x_2j, x_2j+1), split into consecutive sections
             for the position axes (t, y, x): pair j in section a with n_a pairs, at index
             k inside it, turns by angle pos_a * theta_k, theta_k = base^(-k / n_a):
               (x_2j, x_2j+1) -> (x_2j cos - x_2j+1 sin, x_2j sin + x_2j+1 cos)
  prep       q' = rope(rms_norm(q, gamma_q)), k' = rope(rms_norm(k, gamma_k)), v' = v

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
import numpy as np

from .attention import widen


def rms_norm(x, gamma, eps):
    """x [..., D] fp64, gamma [D] -> [..., D] fp64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def rope_angles(pos, sections, base):
    """pos [n, 3] (t, y, x) integers -> angles [n, D/2] fp64 of every rotation pair."""
    pos = np.asarray(pos, dtype=np.float64)
    cols = []
    for a, n_a in enumerate(sections):
        k = np.arange(n_a, dtype=np.float64)
        theta = np.power(float(base), -k / n_a) if n_a else np.zeros(0)
        cols.append(pos[:, a:a + 1] * theta[None, :])
    return np.concatenate(cols, axis=1)


def rope(x, pos, sections, base):
    """x [n, H, D] fp64, pos [n, 3] -> rotated [n, H, D] fp64 (interleaved pairs)."""
    x = np.asarray(x, dtype=np.float64)
    if 2 * sum(sections) != x.shape[-1]:
        raise ValueError("the sections must cover head_dim / 2 pairs")
    ang = rope_angles(pos, sections, base)[:, None, :]          # [n, 1, D/2]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def prep_qkv(qkv, pos, gamma_q, gamma_k, eps, sections, base, dtype):
    """qkv [n][3][H][D] storage array -> (q', k', v) fp64 [n][H][D] each."""
    q = widen(qkv[:, 0], dtype)
    k = widen(qkv[:, 1], dtype)
    v = widen(qkv[:, 2], dtype)
    qn = rope(rms_norm(q, gamma_q, eps), pos, sections, base)
    kn = rope(rms_norm(k, gamma_k, eps), pos, sections, base)
    return qn, kn, v
