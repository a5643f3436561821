"""The query of one new token per sequence, and rotary frequencies with YaRN
(oracle; test only).

DeepSeek-V2 paper (Chinese translation):
  * section 2.1.2, the paragraph on compressing the query as well: the
    query's latent is the down-projection c_Q = W_DQ h (W_DQ of shape
    d'_c x d) and the content query is its up-projection q^C = W_UQ c_Q
    (W_UQ of shape d_h n_h x d'_c);
  * section 2.1.3 (decoupled RoPE): the rotary query of every head is
    q^R = RoPE(W_QR c_Q), W_QR of shape d_h^R n_h x d'_c, rotated at the
    token's position;
  * section 3.1.2 (model hyper-parameters): d'_c = 1536, and an extra RMS norm
    follows each compressed latent vector (so c_Q is normed, like c_KV);
  * section 3.1.4 (long-context extension): YaRN is applied to the decoupled
    rotary key (and so to the rotary query it is scored against) with scale
    s = 40, alpha = 1, beta = 32, extending a 4K context to 160K.

The pages name YaRN but do not restate it; the frequencies follow the YaRN
paper they cite (Peng et al., 2023), its "by parts" interpolation: a feature
pair whose wavelength is short against the original context keeps its
frequency, one whose wavelength is long is interpolated by s, and the pairs in
between are blended linearly in the number of turns they make within the
original context. The length-scaling factor of the softmax (section 3.1.4)
is not part of the query: it multiplies the softmax scale.
Everything is float64.
"""

import math

import numpy as np

from .append import rms_norm, rope_with


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def rope_frequencies(d_rope, base, yarn_scale=1.0, yarn_alpha=1.0, yarn_beta=32.0, orig_ctx=4096):
    """Angle per position of each feature pair (2i, 2i + 1), i < d_rope / 2.

    RoPE: theta_i = base^(-2i / d_rope). YaRN (scale s > 1): the pair makes
    r_i = orig_ctx / (2 pi / theta_i) turns over the original context; with
    g = clamp((r_i - alpha) / (beta - alpha), 0, 1) its frequency becomes
    (1 - g) theta_i / s + g theta_i. s = 1 leaves every frequency unchanged.
    """
    i = np.arange(d_rope // 2, dtype=np.float64)
    theta = float(base) ** (-2.0 * i / d_rope)
    s = float(yarn_scale)
    if s == 1.0:
        return theta
    turns = float(orig_ctx) * theta / (2.0 * math.pi)
    g = np.clip((turns - yarn_alpha) / (yarn_beta - yarn_alpha), 0.0, 1.0)
    return (1.0 - g) * theta / s + g * theta


def query_path(h, w_dq, w_uq, w_qr, positions, eps, freqs, n_heads, gain=None):
    """(c_q [B, d'_c], q_nope [B, H, d_nope], q_rope [B, H, d_rope]).

    h [B, d] hidden states, w_dq [d'_c, d], w_uq [H * d_nope, d'_c] (rows
    grouped by head), w_qr [H * d_rope, d'_c], positions [B], freqs [d_rope/2]
    (rope_frequencies), gain [d'_c] of the norm or None (1).
    """
    h = _f64(h)
    B = h.shape[0]
    c_q = rms_norm(h @ _f64(w_dq).T, eps, gain)
    q_nope = (c_q @ _f64(w_uq).T).reshape(B, n_heads, -1)
    q_r = (c_q @ _f64(w_qr).T).reshape(B, n_heads, -1)
    pos = np.asarray(positions, dtype=np.float64)[:, None] * np.ones((1, n_heads))
    q_rope = rope_with(q_r, pos, freqs)
    return c_q, q_nope, q_rope
