"""The cache entry of one new token (oracle; test only).

DeepSeek-V2 paper (Chinese translation):
  * section 2.1.2 (low-rank key-value joint compression): the cached latent
    of token t is the down-projection of its hidden state, c_KV = W_DKV h,
    with W_DKV of shape d_c x d;
  * section 2.1.3 (decoupled RoPE): the shared rotary key is
    k_R = RoPE(W_KR h), with W_KR of shape d_R x d, rotated at the token's
    position;
  * section 3.1.2 (model hyper-parameters): an extra RMS norm follows the
    compressed latent vector.

The pages give no formula for the norm or the rotation. Readings taken: the
norm is x / sqrt(mean(x^2) + eps) times an optional per-feature gain (the
pages name no gain; none means 1); the rotation pairs features (2i, 2i + 1)
with angle position * base^(-2i / d_R), as in the RoPE paper the pages cite.
Everything is float64.
"""

import numpy as np

from .e4m3 import E4M3_MAX, encode_e4m3


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def rms_norm(x, eps, gain=None):
    """x / sqrt(mean(x^2) + eps) over the last axis, times gain if given."""
    x = _f64(x)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return y if gain is None else y * _f64(gain)


def rope(x, position, base):
    """Rotate the pairs (x[2i], x[2i+1]) of the last axis by position * base^(-2i/d)."""
    x = _f64(x)
    d = x.shape[-1]
    inv_freq = float(base) ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    ang = np.asarray(position, dtype=np.float64)[..., None] * inv_freq
    cos, sin = np.cos(ang), np.sin(ang)
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * cos - x[..., 1::2] * sin
    out[..., 1::2] = x[..., 0::2] * sin + x[..., 1::2] * cos
    return out


def rope_with(x, position, freqs):
    """Rotate the pairs (x[2i], x[2i+1]) of the last axis by position * freqs[i]."""
    x = _f64(x)
    ang = np.asarray(position, dtype=np.float64)[..., None] * _f64(freqs)
    cos, sin = np.cos(ang), np.sin(ang)
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * cos - x[..., 1::2] * sin
    out[..., 1::2] = x[..., 0::2] * sin + x[..., 1::2] * cos
    return out


def append_entry(h, w_dkv, w_kr, positions, eps, base, gain=None, freqs=None):
    """(c_kv [B, d_c], k_rope [B, d_R]) of one new token per sequence.

    h [B, d] hidden states, w_dkv [d_c, d], w_kr [d_R, d], positions [B].
    freqs [d_R / 2]: the rotary frequencies when they are not base^(-2i/d_R)
    (a length-extended model rotates its keys with the YaRN frequencies of
    oracle.query.rope_frequencies, as its queries).
    """
    h = _f64(h)
    c_kv = rms_norm(h @ _f64(w_dkv).T, eps, gain)
    y = h @ _f64(w_kr).T
    k_rope = rope(y, positions, base) if freqs is None else rope_with(y, positions, freqs)
    return c_kv, k_rope


def quantise_entry(c_kv):
    """The e4m3 cache form of latent rows: per row, scale = absmax / 448 (an
    all-zero row gets 1) and code = e4m3(c / scale), rounded to nearest even
    and saturating. Returns (codes uint8, scale float64)."""
    c = _f64(c_kv)
    amax = np.max(np.abs(c), axis=-1)
    scale = np.where(amax > 0, amax / E4M3_MAX, 1.0)
    return encode_e4m3(c / scale[..., None]), scale
