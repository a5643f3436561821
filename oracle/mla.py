"""Plain float64 MLA decode, non-absorbed form (oracle; test infrastructure only).

Source: DeepSeek-V2 paper (Chinese translation), section 2.1.
  * 2.1.1 (standard MHA): per-head attention; output projection; an MHA cache
    holds 2 * n_h * d_h elements per token per layer.
  * 2.1.2 (low-rank key-value joint compression): the cache holds the latent
    c_KV (width d_c); keys and values are its up-projections
    k^C = W_UK c_KV and v^C = W_UV c_KV with W_UK, W_UV in R^{(d_h n_h) x d_c};
    W_UK can be absorbed into the query side and W_UV into the output side.
  * 2.1.3 (decoupled RoPE): one rotary key k^R (width d_h^R) shared by all
    heads is cached beside c_KV; each head's query and key are the
    concatenations [q^C; q^R] and [k^C; k^R]; cache = (d_c + d_h^R) elements
    per token per layer.
  * 2.1.4 / Table 1 caption: that cache equals GQA with 2.25 groups when
    d_c = 4 d_h and d_h^R = d_h / 2.

The display equations of these sections did not survive on the page; the
formulas below are the plainest reading of the surviving prose (matrix shapes,
concatenation, absorption), i.e. textbook scaled softmax attention per head.

Conventions (array layouts are this oracle's own):
  c_kv   [L, d_c]           latent rows of one sequence
  k_rope [L, d_r]           rotary key rows (RoPE already applied)
  q_nope [H, d_nope]        per-head content query q^C
  q_rope [H, d_r]           per-head rotary query q^R (RoPE already applied)
  w_uk   [H, d_nope, d_c]   W_UK with its (d_h n_h) rows grouped by head
  w_uv   [H, d_v, d_c]      W_UV likewise
  sm_scale                  softmax scale (1/sqrt(d_nope + d_r) unless a
                            length-extension factor is folded in)
LSE values are natural-log log-sum-exp of the scaled scores.
"""

import numpy as np

from .e4m3 import decode_e4m3


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def attend_nonabsorbed(c_kv, k_rope, q_nope, q_rope, w_uk, w_uv, sm_scale):
    """Attention of one query token over one sequence's cache, all heads.

    Non-absorbed form (section 2.1.2 + 2.1.3): up-project every cached latent
    to per-head keys and values, concatenate the shared rotary key, then run
    softmax attention per head. Returns (o [H, d_v], lse [H]).
    An empty cache gives o = 0 and lse = -inf.
    """
    c_kv, k_rope = _f64(c_kv), _f64(k_rope)
    q_nope, q_rope = _f64(q_nope), _f64(q_rope)
    w_uk, w_uv = _f64(w_uk), _f64(w_uv)
    H, d_nope, d_c = w_uk.shape
    d_v = w_uv.shape[1]
    L = c_kv.shape[0]
    o = np.zeros((H, d_v))
    lse = np.full(H, -np.inf)
    if L == 0:
        return o, lse
    # k^C_t = W_UK c_KV_t and v^C_t = W_UV c_KV_t, with the (d_h n_h)-row
    # matrices split into n_h heads afterwards.
    k_c = (c_kv @ w_uk.reshape(H * d_nope, d_c).T).reshape(L, H, d_nope)
    v_c = (c_kv @ w_uv.reshape(H * d_v, d_c).T).reshape(L, H, d_v)
    for h in range(H):
        k = np.concatenate([k_c[:, h, :], k_rope], axis=1)   # [k^C; k^R]
        q = np.concatenate([q_nope[h], q_rope[h]])            # [q^C; q^R]
        s = sm_scale * (k @ q)                                 # scores [L]
        m = s.max()
        e = np.exp(s - m)
        z = e.sum()
        o[h] = (e / z) @ v_c[:, h, :]
        lse[h] = m + np.log(z)
    return o, lse


def attend_absorbed(c_kv, k_rope, q_nope, q_rope, w_uk, w_uv, sm_scale):
    """The same attention in absorbed form (section 2.1.2, last sentences).

    W_UK moves to the query side (q_lat = W_UK^T q^C per head) and W_UV to
    the output side (o = W_UV o_lat), so keys and values are never formed.
    Used only to pin the non-absorbed oracle; returns (o, lse, o_lat).
    """
    c_kv, k_rope = _f64(c_kv), _f64(k_rope)
    q_nope, q_rope = _f64(q_nope), _f64(q_rope)
    w_uk, w_uv = _f64(w_uk), _f64(w_uv)
    H, _, d_c = w_uk.shape
    d_v = w_uv.shape[1]
    L = c_kv.shape[0]
    o = np.zeros((H, d_v))
    o_lat = np.zeros((H, d_c))
    lse = np.full(H, -np.inf)
    if L == 0:
        return o, lse, o_lat
    for h in range(H):
        q_lat = w_uk[h].T @ q_nope[h]
        s = sm_scale * (c_kv @ q_lat + k_rope @ q_rope[h])
        m = s.max()
        e = np.exp(s - m)
        z = e.sum()
        o_lat[h] = (e / z) @ c_kv
        o[h] = w_uv[h] @ o_lat[h]
        lse[h] = m + np.log(z)
    return o, lse, o_lat


def token_rows(b, length, seq_stride=None, block_table=None, page_size=0):
    """Physical row index of tokens 0..length-1 of sequence b.

    Contiguous cache: row = b * seq_stride + j.
    Paged cache: token j lives in logical page j // page_size, which the
    block table maps to a physical page; row = page * page_size + j % page_size.
    """
    j = np.arange(length, dtype=np.int64)
    if page_size == 0:
        return b * int(seq_stride) + j
    bt = np.asarray(block_table, dtype=np.int64)
    return bt[b, j // page_size] * page_size + j % page_size


def gather_rows(cache, b, length):
    """(c_kv [L, d_c], k_rope [L, d_r]) in float64 for sequence b.

    `cache` is a dict:
      kind "dense": rows [R, d_c + d_r] (float values, c_KV then k^R)
      kind "fp8":   codes [R, d_c] uint8 (e4m3), scale [R] float,
                    rope [R, d_r] float; c_KV = decode(code) * scale
      plus d_c, and either seq_stride (contiguous) or block_table and
      page_size (paged).
    """
    rows = token_rows(b, length, cache.get("seq_stride"), cache.get("block_table"),
                      cache.get("page_size", 0))
    d_c = cache["d_c"]
    if cache["kind"] == "dense":
        r = _f64(np.asarray(cache["rows"])[rows])
        return r[:, :d_c], r[:, d_c:]
    if cache["kind"] == "fp8":
        codes = np.asarray(cache["codes"])[rows]
        scale = _f64(np.asarray(cache["scale"])[rows])
        return decode_e4m3(codes) * scale[:, None], _f64(np.asarray(cache["rope"])[rows])
    raise ValueError("unknown cache kind %r" % (cache["kind"],))


def decode(q_nope, q_rope, w_uk, w_uv, cache, seq_lens, sm_scale):
    """Batched decode: o [B, H, d_v] and lse [B, H], one sequence at a time."""
    q_nope, q_rope = _f64(q_nope), _f64(q_rope)
    B, H, _ = q_nope.shape
    d_v = np.shape(w_uv)[1]
    o = np.zeros((B, H, d_v))
    lse = np.zeros((B, H))
    for b in range(B):
        c_kv, k_rope = gather_rows(cache, b, int(seq_lens[b]))
        o[b], lse[b] = attend_nonabsorbed(c_kv, k_rope, q_nope[b], q_rope[b],
                                          w_uk, w_uv, sm_scale)
    return o, lse


def decode_heads(q_nope, q_rope, w_uk, w_uv, cache, seq_lens, sm_scale, b, heads):
    """Outputs of `decode` for sequence b and the listed heads only:
    o [len(heads), d_v], lse [len(heads)] (one gather of the sequence's rows,
    the same attention restricted to those heads). For checks at full size."""
    hs = np.asarray(heads, dtype=np.int64).reshape(-1)
    c_kv, k_rope = gather_rows(cache, b, int(seq_lens[b]))
    return attend_nonabsorbed(c_kv, k_rope, _f64(q_nope)[b, hs], _f64(q_rope)[b, hs],
                              _f64(w_uk)[hs], _f64(w_uv)[hs], sm_scale)


def decode_multi(q_nope, q_rope, w_uk, w_uv, cache, seq_lens, sm_scale, n):
    """Decode of n new tokens per sequence in one pass: o [B n, H, d_v] and
    lse [B n, H]; query row b n + t is token t of sequence b.

    DeepSeek-V3 blog (third page), section 3 "multi-token prediction": the
    model proposes several future tokens at once, so a decode step scores n
    tokens of one sequence together. The pages give no formula; the reading
    here is causal attention: the n tokens' own cache entries are appended
    first (seq_lens[b] counts them), token t sits at position
    seq_lens[b] - n + t and attends to cache rows 0 .. seq_lens[b] - n + t
    (its own included, the later ones masked). A token with no row left
    (seq_lens[b] < n - t) gives o = 0 and lse = -inf. n = 1 is `decode`.
    """
    q_nope, q_rope = _f64(q_nope), _f64(q_rope)
    BN, H, _ = q_nope.shape
    d_v = np.shape(w_uv)[1]
    o = np.zeros((BN, H, d_v))
    lse = np.zeros((BN, H))
    for bv in range(BN):
        b, t = divmod(bv, n)
        length = max(0, int(seq_lens[b]) - (n - 1 - t))
        c_kv, k_rope = gather_rows(cache, b, length)
        o[bv], lse[bv] = attend_nonabsorbed(c_kv, k_rope, q_nope[bv], q_rope[bv], w_uk, w_uv, sm_scale)
    return o, lse


def prefill(q_nope, q_rope, w_uk, w_uv, cache, seq_lens, sm_scale, n):
    """Attention of n new tokens per sequence in the non-absorbed form, as a
    prompt is processed: o [B n, H, d_v], lse [B n, H] (row b n + t = token t).

    DeepSeek-V2 paper, section 2.1.2: keys and values are the up-projections
    k^C = W_UK c_KV and v^C = W_UV c_KV of the cached latents; section 2.1.3:
    each head's key is [k^C; k^R]. Here every cached row of a sequence is
    up-projected once and each head runs causal softmax attention: token t
    (position L_b - n + t) attends to rows 0 .. L_b - n + t, the same masking
    as `decode_multi`, which reaches the same values without ever forming
    per-token key sets. A token with no visible row gives o = 0, lse = -inf.
    """
    q_nope, q_rope = _f64(q_nope), _f64(q_rope)
    w_uk, w_uv = _f64(w_uk), _f64(w_uv)
    BN, H, d_nope = q_nope.shape
    d_v, d_c = w_uv.shape[1], w_uv.shape[2]
    B = BN // n
    o = np.zeros((BN, H, d_v))
    lse = np.full((BN, H), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        c_kv, k_rope = gather_rows(cache, b, L)
        k_c = (c_kv @ w_uk.reshape(H * d_nope, d_c).T).reshape(L, H, d_nope)
        v_c = (c_kv @ w_uv.reshape(H * d_v, d_c).T).reshape(L, H, d_v)
        pos = L - n + np.arange(n)                              # position of each new token
        visible = np.arange(L)[None, :] <= pos[:, None]         # [n, L] causal mask
        rows = slice(b * n, (b + 1) * n)
        for h in range(H):
            k = np.concatenate([k_c[:, h, :], k_rope], axis=1)                     # [L, d_nope + d_r]
            q = np.concatenate([q_nope[rows, h, :], q_rope[rows, h, :]], axis=1)   # [n, d_nope + d_r]
            s = np.where(visible, sm_scale * (q @ k.T), -np.inf)                   # [n, L]
            m = s.max(axis=1, initial=-np.inf)
            has = np.isfinite(m)
            e = np.where(visible, np.exp(s - np.where(has, m, 0.0)[:, None]), 0.0)
            z = e.sum(axis=1)
            zs = np.where(has, z, 1.0)
            o[rows, h] = (e / zs[:, None]) @ v_c[:, h, :]
            lse[rows, h] = np.where(has, m + np.log(zs), -np.inf)
    return o, lse


def decode_one(q_nope, q_rope, w_uk, w_uv, cache, seq_lens, sm_scale, b, h):
    """One (sequence, head) output of `decode`: (o [d_v], lse)."""
    o, lse = decode_heads(q_nope, q_rope, w_uk, w_uv, cache, seq_lens, sm_scale, b, [h])
    return o[0], lse[0]


def lse_merge(o_parts, lse_parts):
    """Merge attention results computed over disjoint token sets.

    o_parts [S, ..., d] are each normalised over their own tokens, lse_parts
    [S, ...] their log-sum-exp. The merged result is the attention over the
    union: LSE = log sum_s exp(LSE_s), o = sum_s exp(LSE_s - LSE) o_s.
    Parts with LSE = -inf (no tokens) contribute nothing; if every part is
    empty the result is o = 0, LSE = -inf.
    """
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    m = lse_parts.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m_safe), 0.0)
    z = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, z, 1.0)), -np.inf)
    wn = np.where(finite, w / np.where(finite, z, 1.0), 0.0)
    o = (wn[..., None] * o_parts).sum(axis=0)
    return o, lse


def attend_split(c_kv, k_rope, q_nope, q_rope, w_uk, w_uv, sm_scale, bounds):
    """Attention over token ranges [bounds[i], bounds[i+1]) merged by LSE."""
    parts_o, parts_l = [], []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        o, l = attend_nonabsorbed(c_kv[lo:hi], k_rope[lo:hi], q_nope, q_rope,
                                  w_uk, w_uv, sm_scale)
        parts_o.append(o)
        parts_l.append(l)
    return lse_merge(np.stack(parts_o), np.stack(parts_l))


# --- closed forms (section 2.1.1, 2.1.3, 2.1.4 and Table 1 caption) ---------

def cache_elements_per_token(d_c, d_rope, layers=1):
    """MLA cache: (d_c + d_h^R) * l elements per token (section 2.1.3)."""
    return (d_c + d_rope) * layers


def mha_elements_per_token(n_h, d_h, layers=1):
    """MHA cache: 2 * n_h * d_h * l elements per token (section 2.1.1)."""
    return 2 * n_h * d_h * layers


def gqa_equivalent_groups(d_c, d_rope, d_h):
    """Number of GQA groups whose cache (2 n_g d_h per layer) equals MLA's."""
    return (d_c + d_rope) / (2.0 * d_h)


def kv_reduction_vs_gqa_model(d_c, d_rope, mla_layers, mla_bits,
                              n_groups, d_h, gqa_layers, gqa_bits):
    """1 - (MLA cache bits per token) / (GQA cache bits per token), all layers."""
    mla = cache_elements_per_token(d_c, d_rope, mla_layers) * mla_bits
    gqa = 2 * n_groups * d_h * gqa_layers * gqa_bits
    return 1.0 - mla / gqa
