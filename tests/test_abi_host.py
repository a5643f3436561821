"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments with the documented status before any GPU
work is enqueued. No kernel is launched here."""

import ctypes
import os
import re

import pytest
import torch

import mla_latent_kv_28_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

# The argument-error cases below pass fake (never dereferenced) pointers. On a
# machine with a GPU a validation bug could turn one into a launch, so they run
# on GPU-less hosts only.
no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="fake-pointer cases run without a GPU")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mla.LIB_PATH):
        from mla_latent_kv_28_amd import build
        build.build()
    return mla.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("mla_absorb_q", "mla_decode", "mla_combine", "mla_out_proj"):
        assert n in names
    assert set(names) == set(mla.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), n


def test_time_next_launch_host_side(L):
    # setting (and clearing) the event pair needs no GPU; a pair is only
    # consumed by a launch, so the test leaves none pending
    assert L.mla_time_next_launch(None, None) == 0
    assert mla.mla_time_next_launch(None, None) == 0


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = mla.status_string(code)
        assert s and s != "unknown status"
    assert mla.status_string(-99) == "unknown status"
    assert mla.last_hip_error() == 0


def test_split_chunk(L):
    assert mla.mla_split_chunk(4096, 8) == 512
    assert mla.mla_split_chunk(131072, 64) == 2048
    assert mla.mla_split_chunk(100, 3) == 64          # ceil(100/3) = 34 -> 64
    assert mla.mla_split_chunk(1, 1) == 32
    assert mla.mla_split_chunk(0, 4) == 0
    assert mla.mla_split_chunk(100, 0) == 0


def test_suggest_splits(L):
    assert mla.mla_suggest_splits(32, 4096, 0, 256) == 8       # 256 items of 512 tokens
    assert mla.mla_suggest_splits(4, 131072, 0, 256) == 64     # 2048-token chunks
    assert mla.mla_suggest_splits(512, 4096, 0, 256) == 1
    assert mla.mla_suggest_splits(1, 100, 0, 256) == 1         # chunks of at least 256
    assert mla.mla_suggest_splits(0, 100, 0, 256) == 1
    s = mla.mla_suggest_splits(64, 32768, 64 * 16640, 256)
    assert 1 <= s <= 1024 and mla.mla_split_chunk(32768, s) >= 256
    # 64 sequences averaging half of 32768 tokens: 14 splits of 2368 tokens
    # make about 480 non-empty items, two full rounds of 256
    assert s == 14


DSV2 = mla.Dims(128, 512, 64, 128, 128)
TINY = mla.Dims(4, 32, 16, 32, 32)
P = 1 << 20          # a fake, aligned, non-null address: never dereferenced


def _cache(**kw):
    c = dict(dtype=mla.BF16, latent=P, rope=None, scale=None, row_stride=576, rope_stride=0,
             page_size=0, seq_stride=4096, block_table=None, max_pages_per_seq=0)
    c.update(kw)
    return mla.KVCache(*[c[f] for f, _ in mla.KVCache._fields_])


def _decode(L, dims=DSV2, batch=1, q=P, cache=None, lens=P, max_len=4096, scale=0.07, splits=1,
            out=P, lse=P, out_dtype=mla.BF16):
    cache = _cache() if cache is None else cache
    d = ctypes.byref(dims) if dims is not None else None
    return L.mla_decode(d, batch, q, ctypes.byref(cache), lens, max_len, scale, splits, out, lse,
                        out_dtype, None)


@no_gpu
def test_decode_argument_errors(L):
    assert L.mla_decode(None, 1, P, None, P, 1, 1.0, 1, P, P, 1, None) == -1
    assert _decode(L, batch=-1) == -2
    assert _decode(L, max_len=-1) == -2
    assert _decode(L, splits=0) == -2
    assert _decode(L, scale=float("nan")) == -2
    assert _decode(L, dims=mla.Dims(64, 512, 64, 128, 128)) == -4
    assert _decode(L, cache=_cache(dtype=7)) == -3
    assert _decode(L, cache=_cache(dtype=mla.F32)) == -3          # f32 cache needs the tiny shape
    assert _decode(L, dims=TINY, cache=_cache(dtype=mla.BF16, row_stride=48, seq_stride=64),
                   max_len=64) == -3
    assert _decode(L, cache=_cache(row_stride=1 << 24)) == -4      # rows beyond 2^24 bytes
    assert _decode(L, out_dtype=mla.FP8_E4M3) == -3
    assert _decode(L, q=None) == -1
    assert _decode(L, lens=None) == -1
    assert _decode(L, out=None) == -1
    assert _decode(L, lse=None) == -1
    assert _decode(L, cache=_cache(latent=None)) == -1
    assert _decode(L, cache=_cache(dtype=mla.FP8_E4M3, row_stride=512, rope=P, scale=None,
                                   rope_stride=64)) == -1
    assert _decode(L, cache=_cache(page_size=64, block_table=None, max_pages_per_seq=64)) == -1
    assert _decode(L, cache=_cache(page_size=48, block_table=P, max_pages_per_seq=100)) == -2
    assert _decode(L, cache=_cache(page_size=64, block_table=P, max_pages_per_seq=63)) == -2
    assert _decode(L, cache=_cache(seq_stride=4095)) == -2
    assert _decode(L, cache=_cache(row_stride=575)) == -2
    assert _decode(L, cache=_cache(row_stride=580)) == -5          # rows must stay 16-byte aligned
    assert _decode(L, q=P + 2) == -5
    assert _decode(L, out=P + 8) == -5
    assert _decode(L, cache=_cache(latent=P + 4)) == -5
    assert _decode(L, batch=0) == 0                                 # empty batch: nothing to do
    # chunks longer than 2^17 tokens: the fixed-reference softmax bound no longer holds
    long_cache = _cache(seq_stride=1 << 18)
    assert _decode(L, cache=long_cache, max_len=(1 << 17) + 1) == -4
    assert _decode(L, cache=long_cache, max_len=1 << 18) == -4
    assert _decode(L, cache=_cache(seq_stride=300000), max_len=300000, splits=2) == -4   # 150016 > 2^17
    assert mla.mla_split_chunk((1 << 17) + 1, 2) <= (1 << 17)        # two splits would be accepted


@no_gpu
def test_decode_multi_argument_errors(L):
    def multi(n, batch=1, splits=1, **kw):
        cache = _cache(**kw)
        return L.mla_decode_multi(ctypes.byref(DSV2), batch, n, P, ctypes.byref(cache), P, 4096, 0.07, splits,
                                  P, P, mla.BF16, None)
    assert L.mla_decode_multi(None, 1, 2, P, None, P, 1, 1.0, 1, P, P, 1, None) == -1
    assert multi(0) == -2                                # at least one token per sequence
    assert multi(-3) == -2
    assert multi(2, batch=-1) == -2
    assert multi(1 << 16, batch=1 << 15) == -2           # 2^31 query rows
    assert multi(1 << 12, batch=1 << 10, splits=1 << 9) == -2   # rows x splits beyond 2^31
    assert multi(4, batch=0) == 0                        # no sequences: nothing to do
    assert multi(4, row_stride=580) == -5                # the decode's own checks apply
    assert multi(4, seq_stride=4095) == -2


@no_gpu
def test_absorb_combine_outproj_argument_errors(L):
    d = ctypes.byref(DSV2)
    assert L.mla_absorb_q(None, 1, P, P, P, P, mla.BF16, None) == -1
    assert L.mla_absorb_q(d, -1, P, P, P, P, mla.BF16, None) == -2
    assert L.mla_absorb_q(d, 1, P, P, P, P, mla.F32, None) == -3
    assert L.mla_absorb_q(d, 1, P, None, P, P, mla.BF16, None) == -1
    assert L.mla_absorb_q(d, 1, P, P, P + 2, P, mla.BF16, None) == -5
    assert L.mla_absorb_q(ctypes.byref(mla.Dims(128, 512, 64, 64, 128)), 1, P, P, P, P,
                          mla.BF16, None) == -4
    assert L.mla_absorb_q(d, 0, None, None, None, None, mla.BF16, None) == 0

    assert L.mla_combine(None, 1, 2, P, mla.F32, P, P, P, mla.F32, None) == -1
    assert L.mla_combine(d, 1, 0, P, mla.F32, P, P, P, mla.F32, None) == -2
    assert L.mla_combine(d, 1, 2000, P, mla.F32, P, P, P, mla.F32, None) == -4
    assert L.mla_combine(d, 1, 2, P, mla.F32, P, P, P, mla.FP8_E4M3, None) == -3
    assert L.mla_combine(d, 1, 2, P, mla.FP8_E4M3, P, P, P, mla.F32, None) == -3
    assert L.mla_combine(d, 1, 2, None, mla.BF16, P, P, P, mla.F32, None) == -1
    assert L.mla_combine(d, 1, 2, P + 4, mla.F32, P, P, P, mla.F32, None) == -5

    assert L.mla_out_proj(None, 1, P, mla.BF16, P, mla.BF16, P, mla.BF16, None) == -1
    assert L.mla_out_proj(d, 1, P, mla.BF16, P, mla.F32, P, mla.BF16, None) == -3
    assert L.mla_out_proj(d, 1, P, mla.FP8_E4M3, P, mla.BF16, P, mla.BF16, None) == -3
    assert L.mla_out_proj(ctypes.byref(TINY), 1, P, mla.BF16, P, mla.F32, P, mla.F32, None) == -3
    assert L.mla_out_proj(d, 1, None, mla.BF16, P, mla.BF16, P, mla.BF16, None) == -1
    assert L.mla_out_proj(d, 1, P, mla.BF16, P, mla.BF16, P + 2, mla.BF16, None) == -5
    assert L.mla_out_proj(d, 0, None, mla.BF16, None, mla.BF16, None, mla.BF16, None) == 0


@no_gpu
def test_combine_out_proj_argument_errors(L):
    d = ctypes.byref(DSV2)
    f = L.mla_combine_out_proj
    assert f(None, 1, 2, P, mla.BF16, P, P, mla.BF16, P, mla.BF16, P, None) == -1
    assert f(d, -1, 2, P, mla.BF16, P, P, mla.BF16, P, mla.BF16, P, None) == -2
    assert f(d, 1, 0, P, mla.BF16, P, P, mla.BF16, P, mla.BF16, P, None) == -2
    assert f(ctypes.byref(TINY), 1, 2, P, mla.BF16, P, P, mla.BF16, P, mla.BF16, P, None) == -4
    assert f(d, 1, 2, P, mla.F32, P, P, mla.BF16, P, mla.BF16, P, None) == -3      # bf16 partials only
    assert f(d, 1, 2, P, mla.BF16, P, P, mla.F32, P, mla.BF16, P, None) == -3      # bf16 weights only
    assert f(d, 1, 2, P, mla.BF16, P, P, mla.BF16, P, mla.FP8_E4M3, P, None) == -3
    assert f(d, 1, 65, P, mla.BF16, P, P, mla.BF16, P, mla.BF16, P, None) == -4      # at most 64 splits
    assert f(d, 1, 2, None, mla.BF16, P, P, mla.BF16, P, mla.BF16, P, None) == -1
    assert f(d, 1, 2, P, mla.BF16, P, None, mla.BF16, P, mla.BF16, P, None) == -1
    assert f(d, 1, 2, P, mla.BF16, P, P, mla.BF16, P + 8, mla.BF16, P, None) == -5
    assert f(d, 0, 2, None, mla.BF16, None, None, mla.BF16, None, mla.BF16, None, None) == 0


def test_binding_refuses_host_tensors(L):
    # the binding never hands a host pointer to the library
    x = torch.zeros(4)
    with pytest.raises(TypeError):
        mla.mla_absorb_q(TINY, 1, x, x, x, x, mla.F32)


@no_gpu
def test_cache_append_argument_errors(L):
    d = ctypes.byref(DSV2)
    ws = mla.mla_cache_append_workspace(DSV2, 4, 5120)
    assert ws == 5 * 4 * 576 * 4                      # 1024-wide contraction parts of the hidden size

    def f(dims=d, batch=4, hidden=5120, h=P, w1=P, w2=P, gain=None, dtype=mla.BF16, eps=1e-6, base=1e4,
          pos=P, cache=None, work=P, work_bytes=ws, rope=None):
        cache = _cache(seq_stride=64) if cache is None else cache
        rope = mla.Rope(base, 1.0, 1.0, 32.0, 4096) if rope is None else rope
        return L.mla_cache_append(dims, batch, hidden, h, w1, w2, gain, dtype, eps, ctypes.byref(rope), pos,
                                  ctypes.byref(cache), work, work_bytes, None)
    assert f(dims=None) == -1
    assert f(batch=-1) == -2
    assert f(hidden=5128) == -2                       # whole 16-wide k steps
    assert f(eps=-1.0) == -2 and f(base=0.0) == -2 and f(eps=float("nan")) == -2
    assert f(dims=ctypes.byref(mla.Dims(64, 512, 64, 128, 128))) == -4
    assert f(dtype=mla.F32) == -3                     # bf16 inputs for this shape
    assert f(cache=_cache(dtype=mla.F32, seq_stride=64)) == -3
    assert f(dims=ctypes.byref(TINY), hidden=128, dtype=mla.F32) == -3      # the tiny shape takes an f32 cache
    assert f(h=None) == -1 and f(pos=None) == -1 and f(work=None) == -1
    assert f(work_bytes=ws - 4) == -2
    assert f(cache=_cache(dtype=mla.FP8_E4M3, row_stride=512, seq_stride=64)) == -1   # no rope / scale
    assert f(cache=_cache(page_size=48, block_table=P, max_pages_per_seq=4)) == -2
    assert f(cache=_cache(page_size=64, block_table=None, max_pages_per_seq=4)) == -1
    assert f(cache=_cache(row_stride=575, seq_stride=64)) == -2
    assert f(h=P + 2) == -5 and f(work=P + 4) == -5
    assert f(batch=0, h=None, w1=None, w2=None, pos=None, work=None) == 0
    # rotary parameters: YaRN needs s >= 1, alpha < beta and an original context
    assert f(rope=mla.Rope(1e4, 0.5, 1.0, 32.0, 4096)) == -2
    assert f(rope=mla.Rope(1e4, 40.0, 32.0, 32.0, 4096)) == -2
    assert f(rope=mla.Rope(1e4, 40.0, 1.0, 32.0, 0)) == -2
    assert f(rope=mla.Rope(float("inf"), 1.0, 1.0, 32.0, 4096)) == -2
    assert L.mla_cache_append(d, 4, 5120, P, P, P, None, mla.BF16, 1e-6, None, P,
                              ctypes.byref(_cache(seq_stride=64)), P, ws, None) == -1


@no_gpu
def test_cache_append_noalloc_argument_errors(L):
    # the workspace form's checks, then the scratch limit (8 MiB), all before
    # the scratch address is looked up
    d = ctypes.byref(DSV2)

    def f(dims=d, batch=4, hidden=5120, h=P, w1=P, w2=P, dtype=mla.BF16, pos=P, cache=None):
        cache = _cache(seq_stride=64) if cache is None else cache
        return L.mla_cache_append_noalloc(dims, batch, hidden, h, w1, w2, None, dtype, 1e-6,
                                          ctypes.byref(mla.Rope(1e4, 1.0, 1.0, 32.0, 4096)), pos,
                                          ctypes.byref(cache), None)
    assert f(dims=None) == -1
    assert f(batch=-1) == -2 and f(hidden=5128) == -2
    assert f(dtype=mla.F32) == -3
    assert f(h=None) == -1 and f(pos=None) == -1
    assert f(h=P + 2) == -5
    assert f(batch=729) == -4                        # 729 x 5 x 576 x 4 bytes > 8 MiB
    assert mla.mla_cache_append_workspace(DSV2, 728, 5120) <= (8 << 20)
    assert f(batch=0, h=None, w1=None, w2=None, pos=None) == 0


@no_gpu
def test_o_proj_argument_errors(L):
    d = ctypes.byref(DSV2)
    ws = mla.mla_o_proj_workspace(DSV2, 2, 5120)
    assert ws == 8 * 2 * 5120 * 4                    # fp32 partial sums of 2048-wide contraction parts
    assert mla.mla_o_proj_workspace(TINY, 2, 128) == 0

    def f(dims=d, batch=2, hidden=5120, o=P, w=P, dtype=mla.BF16, out=P, out_dtype=mla.BF16, work=P, nbytes=ws):
        return L.mla_o_proj(dims, batch, hidden, o, w, dtype, out, out_dtype, work, nbytes, None)
    assert f(dims=None) == -1
    assert f(batch=-1) == -2
    assert f(hidden=5120 - 16) == -2                  # 32-feature blocks
    assert f(dtype=mla.F32) == -3 and f(out_dtype=mla.FP8_E4M3) == -3
    assert f(dims=ctypes.byref(TINY), hidden=128, dtype=mla.BF16, out_dtype=mla.F32) == -3
    assert f(dims=ctypes.byref(mla.Dims(8, 512, 64, 128, 128))) == -4
    assert f(o=None) == -1 and f(work=None) == -1
    assert f(nbytes=ws - 4) == -2
    assert f(w=P + 2) == -5 and f(work=P + 4) == -5
    assert f(batch=0, o=None, w=None, out=None, work=None) == 0


@no_gpu
def test_query_proj_argument_errors(L):
    d = ctypes.byref(DSV2)
    ws = mla.mla_query_proj_workspace(DSV2, 4, 5120, 1536)
    # partial sums of W_DQ h (1024-wide contraction parts: 5), plus c_Q in bf16
    # with its rows padded to 32
    assert ws == 5 * 4 * 1536 * 4 + 32 * 1536 * 2
    assert mla.mla_query_proj_workspace(TINY, 4, 128, 256) == 0
    yarn = mla.Rope(1e4, 40.0, 1.0, 32.0, 4096)

    def f(dims=d, batch=4, hidden=5120, dq=1536, h=P, w_dq=P, gain=None, w_uq=P, w_qr=P, dtype=mla.BF16,
          eps=1e-6, rope=yarn, pos=P, qn=P, qr=P, work=P, nbytes=ws):
        return L.mla_query_proj(dims, batch, hidden, dq, h, w_dq, gain, w_uq, w_qr, dtype, eps,
                                None if rope is None else ctypes.byref(rope), pos, qn, qr, work, nbytes, None)
    assert f(dims=None) == -1 and f(rope=None) == -1
    assert f(batch=-1) == -2 and f(hidden=5128) == -2 and f(dq=1000) == -2 and f(eps=-1.0) == -2
    assert f(dims=ctypes.byref(TINY)) == -4 and f(dq=8192) == -4
    assert f(hidden=20496) == -4                           # beyond 16 partial sums of W_DQ h
    assert f(dtype=mla.F32) == -3
    assert f(rope=mla.Rope(1e4, 40.0, 5.0, 5.0, 4096)) == -2
    assert f(h=None) == -1 and f(qr=None) == -1 and f(work=None) == -1 and f(pos=None) == -1
    assert f(nbytes=ws - 4) == -2
    assert f(w_uq=P + 2) == -5 and f(qn=P + 8) == -5
    assert f(batch=0, h=None, w_dq=None, w_uq=None, w_qr=None, pos=None, qn=None, qr=None, work=None) == 0


@no_gpu
def test_read_probe_argument_errors(L):
    assert L.mla_read_probe(P, 0, P, None) == 0            # nothing to read
    assert L.mla_read_probe(P, -16, P, None) == -2
    assert L.mla_read_probe(P, 24, P, None) == -2          # not a multiple of 16
    assert L.mla_read_probe(None, 1 << 20, P, None) == -1
    assert L.mla_read_probe(P, 1 << 20, None, None) == -1
    assert L.mla_read_probe(P + 8, 1 << 20, P, None) == -5


@no_gpu
def test_prefill_argument_errors(L):
    def pre(n=4, batch=1, max_len=4096, ws=1 << 40, dims=DSV2, scale=0.07, **kw):
        cache = _cache(**kw)
        d = ctypes.byref(dims) if dims is not None else None
        return L.mla_prefill(d, batch, n, P, P, ctypes.byref(cache), P, max_len, P, P, scale, P, P, P, ws, None)
    need = L.mla_prefill_workspace(ctypes.byref(DSV2), 2, 1000)
    assert need == 2 * 2 * 128 * 1024 * 128 * 2          # K^C and V^C, 1000 tokens padded to 1024
    assert L.mla_prefill_workspace(ctypes.byref(TINY), 2, 1000) == 0
    assert pre(dims=None) == -1
    assert pre(n=0) == -2
    assert pre(batch=-1) == -2
    assert pre(max_len=-1) == -2
    assert pre(scale=float("inf")) == -2
    assert pre(dims=TINY) == -4
    assert pre(dtype=mla.FP8_E4M3) == -3                 # bf16 caches only
    assert pre(dtype=mla.F32) == -3
    assert pre(batch=0) == 0
    assert pre(ws=need // 2) == -2                       # workspace too small for 1 x 4096 tokens
    assert pre(max_len=1000, batch=2, ws=need - 16) == -2
    assert pre(row_stride=580) == -5
    assert pre(seq_stride=4095) == -2
    assert pre(page_size=48, block_table=P, max_pages_per_seq=100) == -2
    assert pre(latent=None) == -1
