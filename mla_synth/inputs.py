"""Seeded input generators for the MLA decode workloads.

Shapes follow the DeepSeek-V2 paper (Chinese translation), section 3.1.2
(hyperparameters): 128 heads of width 128, latent width d_c = 512, decoupled
rotary width 64, hidden size 5120, parameters initialised with std 0.006.
Trained weights and the deployed service's length distribution are not
available, so every tensor here is synthetic.

Draw order (numpy.random.default_rng(seed), PCG64, float64 draws, rounded to
the storage dtype with round-to-nearest-even at the end):

  tiny workload (fp32, 4 heads):
    hidden states h[L, hidden] ~ N(0, 1); then W_DKV[d_c, hidden],
    W_KR[d_r, hidden], W_Q[H*(d_nope+d_r), hidden], W_UK[H, d_nope, d_c],
    W_UV[H, d_v, d_c], each ~ N(0, 1) / sqrt(fan_in).
    c_KV_j = W_DKV h_j; k^R_j = RoPE(W_KR h_j, position j);
    q = W_Q h_{L-1} split per head into q_nope and q_rope (RoPE at L-1).
  DeepSeek-V2-shaped workloads:
    for each sequence b in order: c_KV rows [L_b, d_c] ~ N(0, 1) then
    RMS-normalised (x / sqrt(mean(x^2) + 1e-6), no gain); k^R rows
    [L_b, d_r] ~ N(0, 1) rotated at positions 0..L_b-1;
    then W_Q[H*(d_nope+d_r), hidden] ~ N(0, 0.006^2), hidden states
    h[B, hidden] ~ N(0, 1), q = W_Q h per sequence, q_rope rotated at L_b-1;
    then W_UK, W_UV ~ N(0, 0.006^2).
  Variable lengths and page placement come from a second generator
  default_rng(len_seed): lengths uniform on [lo, hi] inclusive, then one
  permutation of the physical page ids, handed out to the sequences' logical
  pages in order.

RoPE: interleaved pairs (2i, 2i+1), theta_i = base^(-2i/d_r), base 10000,
angles in float64.
"""

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Dims:
    num_heads: int
    d_latent: int
    d_nope: int
    d_rope: int
    d_v: int
    hidden: int

    @property
    def width(self):
        return self.d_latent + self.d_rope


TINY = Dims(num_heads=4, d_latent=32, d_nope=32, d_rope=16, d_v=32, hidden=128)
DSV2 = Dims(num_heads=128, d_latent=512, d_nope=128, d_rope=64, d_v=128, hidden=5120)

# Length-extension factor multiplied into the softmax scale of the long-context
# workload: 0.1 * ln(40) + 1.
LONG_MSCALE = 0.1 * math.log(40.0) + 1.0

WORKLOADS = {
    # batch 1, 64 cached tokens, fp32, 4 heads
    "tiny": dict(dims=TINY, batch=1, seq_len=64, layout="contiguous", dtype="f32", splits=1),
    # DeepSeek-V2 shapes, batch 32, every length 4096, bf16
    "dsv2_b32_l4096": dict(dims=DSV2, batch=32, seq_len=4096, layout="contiguous", dtype="bf16"),
    # batch 64, lengths uniform on [512, 32768], 64-token pages, bf16
    "paged_varlen_b64": dict(dims=DSV2, batch=64, seq_len=("uniform", 512, 32768),
                             layout="paged", page_size=64, dtype="bf16", len_seed=1),
    # batch 4, length 131072, 64 splits, scale times LONG_MSCALE
    "long_b4_l131072": dict(dims=DSV2, batch=4, seq_len=131072, layout="contiguous",
                            dtype="bf16", splits=64, mscale=LONG_MSCALE),
    # batch 128, length 8192, e4m3 latent with per-token fp32 scale, bf16 rope
    "fp8_b128_l8192": dict(dims=DSV2, batch=128, seq_len=8192, layout="contiguous", dtype="fp8"),
}

E4M3_MAX = 448.0


def rope_rotate(x, positions, base=10000.0):
    """Rotate the last dim of x (float64, even width) by RoPE at `positions`.

    x[..., n, d] with positions[n]; interleaved pairs (2i, 2i+1).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    inv = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)          # [d/2]
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def rms_normalise(x, eps=1e-6):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _store(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.float32 if dtype == "f32" else torch.bfloat16)


def quantise_rows_e4m3(rows, d_latent):
    """Split bf16 rows [R, d_c + d_r] into the fp8 cache layout.

    Per row: scale = absmax(c_KV in fp32) / 448 (an all-zero row gets 1),
    code = e4m3(c_KV / scale) with round-to-nearest-even (values clamped to
    +-448 first). The rotary part stays bf16. Returns (codes uint8 [R, d_c],
    scale float32 [R], rope bf16 [R, d_r]).
    """
    c = rows[:, :d_latent].float()
    amax = c.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (c / scale[:, None]).clamp(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    rope = rows[:, d_latent:].to(torch.bfloat16).contiguous()
    return codes, scale.contiguous(), rope


@dataclass
class Inputs:
    name: str
    dims: Dims
    dtype: str                 # "f32" | "bf16" | "fp8" (cache); q and weights are bf16 for fp8
    seq_lens: np.ndarray       # int32 [B]
    sm_scale: float
    q_nope: torch.Tensor       # [B, H, d_nope]
    q_rope: torch.Tensor       # [B, H, d_rope]
    w_uk: torch.Tensor         # [H, d_nope, d_latent]
    w_uv: torch.Tensor         # [H, d_v, d_latent]
    rows: torch.Tensor         # [R, d_latent + d_rope] dense rows (bf16 original for fp8)
    layout: str                # "contiguous" | "paged"
    seq_stride: int = 0        # contiguous: rows per sequence
    page_size: int = 0         # paged: rows per page
    block_table: Optional[np.ndarray] = None   # paged: int32 [B, max_pages]
    codes: Optional[torch.Tensor] = None       # fp8: uint8 [R, d_latent]
    scale: Optional[torch.Tensor] = None       # fp8: float32 [R]
    rope: Optional[torch.Tensor] = None        # fp8: bf16 [R, d_rope]
    splits: int = 0            # suggested split count (0 = choose)
    tokens_per_seq: int = 1    # query rows per sequence (q_* hold batch * n rows)
    extra: dict = field(default_factory=dict)

    @property
    def batch(self):
        return int(self.seq_lens.shape[0])

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    @property
    def compute_dtype(self):
        return "f32" if self.dtype == "f32" else "bf16"

    def cache_bytes(self):
        """Bytes of latent cache the decode must read (valid tokens only)."""
        n = int(self.seq_lens.astype(np.int64).sum())
        if self.dtype == "fp8":
            return n * (self.dims.d_latent + 2 * self.dims.d_rope + 4)
        return n * self.dims.width * (4 if self.dtype == "f32" else 2)


def _lengths(spec, batch, rng_len, override):
    if override is not None:
        lens = np.asarray(override, dtype=np.int64)
        if lens.ndim == 0:
            lens = np.full(batch, int(lens), dtype=np.int64)
        return lens
    if isinstance(spec, tuple):
        _, lo, hi = spec
        return rng_len.integers(lo, hi, size=batch, endpoint=True).astype(np.int64)
    return np.full(batch, int(spec), dtype=np.int64)


def make_inputs(name, seed=0, batch=None, seq_lens=None, layout=None, page_size=None,
                dtype=None, q_scale=1.0, pad_fill=0.0, len_seed=None, sm_scale=None,
                seq_stride=None, tokens_per_seq=1):
    """Build one workload's inputs on the host.

    Overrides (for smaller parity cases and stress variants): batch,
    seq_lens (int or list), layout, page_size, dtype, q_scale (multiplies q
    before rounding; 30 gives peaked attention), pad_fill (value written into
    cache rows that no sequence owns: padding of a contiguous cache and the
    tail of a sequence's last page; NaN checks that masked rows never leak),
    sm_scale, seq_stride, tokens_per_seq (n query rows per sequence, row
    b n + t rotated at position L_b - n + t: the newest n tokens of each
    sequence; DeepSeek-V2 shape only).
    """
    w = dict(WORKLOADS[name])
    dims = w["dims"]
    batch = w["batch"] if batch is None else batch
    layout = w["layout"] if layout is None else layout
    dtype = w["dtype"] if dtype is None else dtype
    page_size = w.get("page_size", 64) if page_size is None else page_size
    len_seed = w.get("len_seed", 1) if len_seed is None else len_seed
    rng_len = np.random.default_rng(len_seed)
    lens = _lengths(w["seq_len"], batch, rng_len, seq_lens)
    batch = int(lens.shape[0])
    if sm_scale is None:
        sm_scale = w.get("mscale", 1.0) / math.sqrt(dims.d_nope + dims.d_rope)
    store = "f32" if dtype == "f32" else "bf16"
    H, dc, dn, dr, dv, hid = (dims.num_heads, dims.d_latent, dims.d_nope, dims.d_rope,
                              dims.d_v, dims.hidden)
    rng = np.random.default_rng(seed)

    # --- per-sequence latent and rotary rows --------------------------------
    seq_rows = []
    if dims == TINY:
        assert batch == 1 and tokens_per_seq == 1, "the tiny workload has one sequence and one query"
        L = int(lens[0])
        h = rng.standard_normal((max(L, 1), hid))
        w_dkv = rng.standard_normal((dc, hid)) / math.sqrt(hid)
        w_kr = rng.standard_normal((dr, hid)) / math.sqrt(hid)
        w_q = rng.standard_normal((H * (dn + dr), hid)) / math.sqrt(hid)
        w_uk = rng.standard_normal((H, dn, dc)) / math.sqrt(dc)
        w_uv = rng.standard_normal((H, dv, dc)) / math.sqrt(dc)
        c = h[:L] @ w_dkv.T
        r = rope_rotate(h[:L] @ w_kr.T, np.arange(L))
        seq_rows.append(np.concatenate([c, r], axis=1))
        q = (h[max(L, 1) - 1] @ w_q.T).reshape(1, H, dn + dr)
        q_nope = q[:, :, :dn]
        q_rope = rope_rotate(q[0, :, dn:], np.full(H, max(L, 1) - 1))[None]
    else:
        for b in range(batch):
            L = int(lens[b])
            c = rms_normalise(rng.standard_normal((L, dc)))
            r = rope_rotate(rng.standard_normal((L, dr)), np.arange(L))
            seq_rows.append(np.concatenate([c, r], axis=1))
        n = int(tokens_per_seq)
        w_q = rng.standard_normal((H * (dn + dr), hid)) * 0.006
        h = rng.standard_normal((batch * n, hid))
        q = (h @ w_q.T).reshape(batch * n, H, dn + dr)
        del w_q
        w_uk = rng.standard_normal((H, dn, dc)) * 0.006
        w_uv = rng.standard_normal((H, dv, dc)) * 0.006
        q_nope = q[:, :, :dn]
        q_rope = np.stack([rope_rotate(q[r, :, dn:],
                                       np.full(H, max(int(lens[r // n]) - n + r % n, 0) if n > 1
                                               else max(int(lens[r]), 1) - 1))
                           for r in range(batch * n)])

    q_nope = q_nope * q_scale
    q_rope = q_rope * q_scale

    # --- place rows in the cache layout ------------------------------------
    width = dc + dr
    fill = np.float64(pad_fill)
    if layout == "contiguous":
        stride = int(lens.max()) if lens.size else 0
        if seq_stride is not None:
            stride = int(seq_stride)
        stride = max(stride, 1)
        rows = torch.empty((batch * stride, width), dtype=torch.float32 if store == "f32"
                           else torch.bfloat16)
        rows.fill_(float(fill))
        for b in range(batch):
            L = int(lens[b])
            if L:
                rows[b * stride: b * stride + L] = _store(seq_rows[b], store)
        block_table = None
    elif layout == "paged":
        pages = [(int(L) + page_size - 1) // page_size for L in lens]
        total = max(sum(pages), 1)
        # One permutation of the physical page ids from the length generator's
        # stream (after the lengths, when they were drawn).
        perm = rng_len.permutation(total)
        max_pages = max(max(pages) if pages else 1, 1)
        block_table = np.zeros((batch, max_pages), dtype=np.int32)
        rows = torch.empty((total * page_size, width), dtype=torch.float32 if store == "f32"
                           else torch.bfloat16)
        rows.fill_(float(fill))
        k = 0
        for b in range(batch):
            L = int(lens[b])
            src = _store(seq_rows[b], store) if L else None
            for p in range(pages[b]):
                phys = int(perm[k])
                k += 1
                block_table[b, p] = phys
                lo, hi = p * page_size, min((p + 1) * page_size, L)
                rows[phys * page_size: phys * page_size + (hi - lo)] = src[lo:hi]
        stride = 0
    else:
        raise ValueError(layout)
    del seq_rows

    inp = Inputs(
        name=name, dims=dims, dtype=dtype, seq_lens=lens.astype(np.int32),
        sm_scale=float(sm_scale),
        q_nope=_store(q_nope, store), q_rope=_store(q_rope, store),
        w_uk=_store(w_uk, store), w_uv=_store(w_uv, store),
        rows=rows, layout=layout, seq_stride=stride if layout == "contiguous" else 0,
        page_size=page_size if layout == "paged" else 0, block_table=block_table,
        splits=w.get("splits", 0), tokens_per_seq=int(tokens_per_seq),
    )
    if dtype == "fp8":
        inp.codes, inp.scale, inp.rope = quantise_rows_e4m3(rows, dc)
    return inp


def oracle_args(inp, fp8_reference="dequantised"):
    """Plain float64 NumPy views of `inp` in the oracle's argument format.

    For the fp8 workload, fp8_reference picks the cache the oracle reads:
    "dequantised" (codes and scales) or "bf16" (the rows before quantisation).
    """
    d = inp.dims
    cache = dict(d_c=d.d_latent)
    if inp.layout == "contiguous":
        cache["seq_stride"] = inp.seq_stride
    else:
        cache["block_table"] = inp.block_table
        cache["page_size"] = inp.page_size
    if inp.dtype == "fp8" and fp8_reference == "dequantised":
        cache.update(kind="fp8", codes=inp.codes.numpy(), scale=inp.scale.numpy(),
                     rope=inp.rope.float().numpy())
    else:
        # float32 holds every bf16 value exactly; the oracle widens to float64
        # after gathering a sequence's rows.
        cache.update(kind="dense", rows=inp.rows.float().numpy())
    return dict(q_nope=inp.q_nope.double().numpy(), q_rope=inp.q_rope.double().numpy(),
                w_uk=inp.w_uk.double().numpy(), w_uv=inp.w_uv.double().numpy(),
                cache=cache, seq_lens=inp.seq_lens, sm_scale=inp.sm_scale)


@dataclass
class AppendInputs:
    """Inputs of the cache entry of one new token per sequence."""
    dims: Dims
    dtype: str                 # "bf16" | "f32" (hidden states and weights)
    h: torch.Tensor            # [B, hidden]
    w_dkv: torch.Tensor        # [d_latent, hidden]
    w_kr: torch.Tensor         # [d_rope, hidden]
    gain: Optional[torch.Tensor]   # [d_latent] or None
    positions: np.ndarray      # int32 [B]
    eps: float = 1e-6
    base: float = 10000.0


def make_append_inputs(dims=DSV2, batch=32, seed=0, max_position=4096, with_gain=False, positions=None):
    """Hidden states N(0, 1); projections N(0, 0.006^2) for the DeepSeek-V2
    shape (the paper's initialisation), N(0, 1) / sqrt(hidden) for the tiny
    shape (stored fp32); an optional gain 1 + N(0, 0.1^2); positions uniform
    on [0, max_position). Draws in that order from default_rng(seed)."""
    rng = np.random.default_rng(seed)
    hid = dims.hidden
    store = "f32" if dims == TINY else "bf16"
    std = 1.0 / math.sqrt(hid) if dims == TINY else 0.006
    h = rng.standard_normal((batch, hid))
    w_dkv = rng.standard_normal((dims.d_latent, hid)) * std
    w_kr = rng.standard_normal((dims.d_rope, hid)) * std
    gain = 1.0 + 0.1 * rng.standard_normal(dims.d_latent) if with_gain else None
    pos = rng.integers(0, max_position, size=batch)
    if positions is not None:
        pos = np.asarray(positions, dtype=np.int64)
    return AppendInputs(dims=dims, dtype=store, h=_store(h, store), w_dkv=_store(w_dkv, store),
                        w_kr=_store(w_kr, store), gain=None if gain is None else _store(gain, store),
                        positions=pos.astype(np.int32))


def make_oproj_inputs(dims=DSV2, batch=32, seed=0):
    """Heads' outputs o [B, H, d_v] ~ N(0, 1) and W_O [hidden, H d_v] ~ N(0, 0.006^2)
    (DeepSeek-V2 shape, bf16) or N(0, 1) / sqrt(H d_v) (tiny, fp32), drawn in
    that order from default_rng(seed). Returns (o, w_o) host tensors."""
    rng = np.random.default_rng(seed)
    k = dims.num_heads * dims.d_v
    store = "f32" if dims == TINY else "bf16"
    o = rng.standard_normal((batch, dims.num_heads, dims.d_v))
    w_o = rng.standard_normal((dims.hidden, k)) * (1.0 / math.sqrt(k) if dims == TINY else 0.006)
    return _store(o, store), _store(w_o, store)


@dataclass
class QueryInputs:
    """Inputs of the query of one new token per sequence."""
    dims: Dims
    d_qlatent: int
    h: torch.Tensor            # [B, hidden] bf16
    w_dq: torch.Tensor         # [d_qlatent, hidden]
    w_uq: torch.Tensor         # [H * d_nope, d_qlatent]
    w_qr: torch.Tensor         # [H * d_rope, d_qlatent]
    gain: Optional[torch.Tensor]   # [d_qlatent] or None
    positions: np.ndarray      # int32 [B]
    eps: float = 1e-6


def make_query_inputs(dims=DSV2, batch=32, seed=0, d_qlatent=1536, max_position=4096, with_gain=False,
                      positions=None):
    """Hidden states N(0, 1); W_DQ, W_UQ, W_QR N(0, 0.006^2) (the paper's
    initialisation; d'_c = 1536 in DeepSeek-V2); an optional norm gain
    1 + N(0, 0.1^2); positions uniform on [0, max_position). Drawn in that
    order from default_rng(seed), stored in bf16."""
    rng = np.random.default_rng(seed)
    H, dn, dr, hid = dims.num_heads, dims.d_nope, dims.d_rope, dims.hidden
    h = rng.standard_normal((batch, hid))
    w_dq = rng.standard_normal((d_qlatent, hid)) * 0.006
    w_uq = rng.standard_normal((H * dn, d_qlatent)) * 0.006
    w_qr = rng.standard_normal((H * dr, d_qlatent)) * 0.006
    gain = 1.0 + 0.1 * rng.standard_normal(d_qlatent) if with_gain else None
    pos = rng.integers(0, max_position, size=batch)
    if positions is not None:
        pos = np.asarray(positions, dtype=np.int64)
    return QueryInputs(dims=dims, d_qlatent=d_qlatent, h=_store(h, "bf16"), w_dq=_store(w_dq, "bf16"),
                       w_uq=_store(w_uq, "bf16"), w_qr=_store(w_qr, "bf16"),
                       gain=None if gain is None else _store(gain, "bf16"), positions=pos.astype(np.int32))
