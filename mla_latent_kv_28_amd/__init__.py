"""Python binding of libmla, the MI355X MLA latent-cache decode library.

Argument marshalling only: every function hands device pointers, sizes and
the current HIP stream to the C ABI declared in include/mla.h; all the
arithmetic runs in the library's HIP kernels. PyTorch supplies device memory
and streams. If libmla.so has not been built, or the tensors are not on a
GPU, the calls raise instead of computing anything elsewhere.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
_STATUS = {0: "MLA_OK", -1: "MLA_ERR_NULL", -2: "MLA_ERR_SHAPE", -3: "MLA_ERR_DTYPE",
           -4: "MLA_ERR_UNSUPPORTED", -5: "MLA_ERR_ALIGN", -6: "MLA_ERR_HIP"}

# Every symbol include/mla.h declares.
EXPORTS = ("mla_absorb_q", "mla_decode", "mla_decode_multi", "mla_combine", "mla_out_proj", "mla_combine_out_proj",
           "mla_split_chunk", "mla_suggest_splits", "mla_status_string", "mla_last_hip_error",
           "mla_time_next_launch", "mla_read_probe",
           "mla_cache_append", "mla_cache_append_workspace", "mla_cache_append_noalloc",
           "mla_o_proj", "mla_o_proj_workspace", "mla_query_proj", "mla_query_proj_workspace",
           "mla_prefill", "mla_prefill_workspace")


class MLAError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = "%s failed: %s (%s)" % (where, _STATUS.get(status, status), status_string(status))
        if status == -6:
            msg += ", hipError_t %d" % last_hip_error()
        super().__init__(msg)


class Dims(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("d_latent", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("d_nope", ctypes.c_int32), ("d_v", ctypes.c_int32)]


class Rope(ctypes.Structure):
    """mla_rope: rotary frequencies, plain RoPE (yarn_scale 1) or YaRN."""
    _fields_ = [("base", ctypes.c_float), ("yarn_scale", ctypes.c_float), ("yarn_alpha", ctypes.c_float),
                ("yarn_beta", ctypes.c_float), ("yarn_orig_ctx", ctypes.c_int32)]


def rope_params(rope):
    """A Rope from a Rope, or from a number (plain RoPE with that base)."""
    if isinstance(rope, Rope):
        return rope
    return Rope(float(rope), 1.0, 1.0, 32.0, 4096)


class KVCache(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("latent", ctypes.c_void_p), ("rope", ctypes.c_void_p),
                ("scale", ctypes.c_void_p), ("row_stride", ctypes.c_int64),
                ("rope_stride", ctypes.c_int64), ("page_size", ctypes.c_int32),
                ("seq_stride", ctypes.c_int64), ("block_table", ctypes.c_void_p),
                ("max_pages_per_seq", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libmla.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmla.so is not built; run `python -m mla_latent_kv_28_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        pd = ctypes.POINTER(Dims)
        L.mla_absorb_q.argtypes = [pd, i32, vp, vp, vp, vp, i32, vp]
        L.mla_decode.argtypes = [pd, i32, vp, ctypes.POINTER(KVCache), vp, i32, f32, i32, vp, vp, i32, vp]
        L.mla_decode_multi.argtypes = [pd, i32, i32, vp, ctypes.POINTER(KVCache), vp, i32, f32, i32, vp, vp, i32,
                                       vp]
        L.mla_combine.argtypes = [pd, i32, i32, vp, i32, vp, vp, vp, i32, vp]
        L.mla_out_proj.argtypes = [pd, i32, vp, i32, vp, i32, vp, i32, vp]
        L.mla_combine_out_proj.argtypes = [pd, i32, i32, vp, i32, vp, vp, i32, vp, i32, vp, vp]
        L.mla_split_chunk.argtypes = [i32, i32]
        L.mla_suggest_splits.argtypes = [i32, i32, i64, i32]
        L.mla_status_string.argtypes = [i32]
        L.mla_status_string.restype = ctypes.c_char_p
        L.mla_last_hip_error.argtypes = []
        L.mla_time_next_launch.argtypes = [vp, vp]
        L.mla_read_probe.argtypes = [vp, i64, vp, vp]
        L.mla_o_proj.argtypes = [pd, i32, i32, vp, vp, i32, vp, i32, vp, i64, vp]
        L.mla_o_proj.restype = i32
        L.mla_o_proj_workspace.argtypes = [pd, i32, i32]
        L.mla_o_proj_workspace.restype = i64
        L.mla_cache_append_workspace.argtypes = [pd, i32, i32]
        L.mla_cache_append_workspace.restype = i64
        pr = ctypes.POINTER(Rope)
        L.mla_cache_append.argtypes = [pd, i32, i32, vp, vp, vp, vp, i32, f32, pr, vp,
                                       ctypes.POINTER(KVCache), vp, i64, vp]
        L.mla_cache_append.restype = i32
        L.mla_cache_append_noalloc.argtypes = [pd, i32, i32, vp, vp, vp, vp, i32, f32, pr, vp,
                                               ctypes.POINTER(KVCache), vp]
        L.mla_cache_append_noalloc.restype = i32
        L.mla_query_proj_workspace.argtypes = [pd, i32, i32, i32]
        L.mla_query_proj_workspace.restype = i64
        L.mla_query_proj.argtypes = [pd, i32, i32, i32, vp, vp, vp, vp, vp, i32, f32, pr, vp, vp, vp, vp, i64, vp]
        L.mla_query_proj.restype = i32
        L.mla_prefill_workspace.argtypes = [pd, i32, i32]
        L.mla_prefill_workspace.restype = i64
        L.mla_prefill.argtypes = [pd, i32, i32, vp, vp, ctypes.POINTER(KVCache), vp, i32, vp, vp, f32, vp, vp, vp,
                                  i64, vp]
        L.mla_prefill.restype = i32
        for name in ("mla_absorb_q", "mla_decode", "mla_decode_multi", "mla_combine", "mla_out_proj", "mla_split_chunk",
                     "mla_suggest_splits", "mla_last_hip_error", "mla_combine_out_proj",
                     "mla_time_next_launch", "mla_read_probe"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def dims_of(d):
    """ctypes Dims from any object with num_heads, d_latent, d_rope, d_nope, d_v."""
    return Dims(d.num_heads, d.d_latent, d.d_rope, d.d_nope, d.d_v)


_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}


def _dev(t, name, dtype=None, numel=None):
    """Device pointer of a GPU tensor (None -> NULL) after layout checks."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a torch tensor on the GPU" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if numel is not None and t.numel() < numel:
        raise ValueError("%s holds %d elements, needs %d" % (name, t.numel(), numel))
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(status, where):
    if status != 0:
        raise MLAError(status, where)


def mla_absorb_q(dims, batch, q_nope, q_rope, w_uk, q_lat, dtype, stream=None):
    d = dims_of(dims)
    td = _TORCH_DTYPE[dtype]
    H = d.num_heads
    st = lib().mla_absorb_q(
        ctypes.byref(d), batch,
        _dev(q_nope, "q_nope", td, batch * H * d.d_nope),
        _dev(q_rope, "q_rope", td, batch * H * d.d_rope),
        _dev(w_uk, "w_uk", td, H * d.d_nope * d.d_latent),
        _dev(q_lat, "q_lat", td, batch * H * (d.d_latent + d.d_rope)),
        dtype, _stream(stream))
    _check(st, "mla_absorb_q")


def kv_cache(dtype, latent, rope=None, scale=None, row_stride=None, rope_stride=0, page_size=0,
             seq_stride=0, block_table=None, max_pages_per_seq=0):
    """An mla_kv_cache describing GPU tensors (kept alive by the caller)."""
    if row_stride is None:
        row_stride = latent.shape[-1]
    return KVCache(dtype, _dev(latent, "latent"), _dev(rope, "rope", torch.bfloat16),
                   _dev(scale, "scale", torch.float32), row_stride, rope_stride, page_size,
                   seq_stride, _dev(block_table, "block_table", torch.int32), max_pages_per_seq)


def mla_decode(dims, batch, q_lat, cache, seq_lens, max_seq_len, sm_scale, num_splits, out, lse,
               out_dtype, stream=None):
    d = dims_of(dims)
    H = d.num_heads
    q_dtype = torch.float32 if cache.dtype == F32 else torch.bfloat16
    parts = num_splits if num_splits > 1 else 1
    st = lib().mla_decode(
        ctypes.byref(d), batch,
        _dev(q_lat, "q_lat", q_dtype, batch * H * (d.d_latent + d.d_rope)),
        ctypes.byref(cache),
        _dev(seq_lens, "seq_lens", torch.int32, batch),
        max_seq_len, float(sm_scale), num_splits,
        _dev(out, "out", _TORCH_DTYPE.get(out_dtype), batch * parts * H * d.d_latent),
        _dev(lse, "lse", torch.float32, batch * parts * H),
        out_dtype, _stream(stream))
    _check(st, "mla_decode")


def mla_decode_multi(dims, batch, tokens_per_seq, q_lat, cache, seq_lens, max_seq_len, sm_scale, num_splits,
                     out, lse, out_dtype, stream=None):
    """mla_decode with tokens_per_seq causal query tokens per sequence:
    q_lat [batch * n, H, 576], out/lse with batch * n rows, seq_lens [batch]."""
    d = dims_of(dims)
    H = d.num_heads
    q_dtype = torch.float32 if cache.dtype == F32 else torch.bfloat16
    parts = num_splits if num_splits > 1 else 1
    rows = batch * max(tokens_per_seq, 0)
    st = lib().mla_decode_multi(
        ctypes.byref(d), batch, tokens_per_seq,
        _dev(q_lat, "q_lat", q_dtype, rows * H * (d.d_latent + d.d_rope)),
        ctypes.byref(cache),
        _dev(seq_lens, "seq_lens", torch.int32, batch),
        max_seq_len, float(sm_scale), num_splits,
        _dev(out, "out", _TORCH_DTYPE.get(out_dtype), rows * parts * H * d.d_latent),
        _dev(lse, "lse", torch.float32, rows * parts * H),
        out_dtype, _stream(stream))
    _check(st, "mla_decode_multi")


def mla_prefill_workspace(dims, batch, max_seq_len):
    return int(lib().mla_prefill_workspace(ctypes.byref(dims_of(dims)), batch, max_seq_len))


def mla_prefill(dims, batch, tokens_per_seq, q_nope, q_rope, cache, seq_lens, max_seq_len, w_uk, w_uv,
                sm_scale, out, lse, workspace, stream=None):
    """Non-absorbed causal attention of tokens_per_seq new tokens per
    sequence: q_* [batch * n, H, *] bf16, out [batch * n, H, d_v] bf16,
    lse [batch * n, H] f32, workspace of mla_prefill_workspace bytes."""
    d = dims_of(dims)
    H = d.num_heads
    rows = batch * max(tokens_per_seq, 0)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().mla_prefill(
        ctypes.byref(d), batch, tokens_per_seq,
        _dev(q_nope, "q_nope", torch.bfloat16, rows * H * d.d_nope),
        _dev(q_rope, "q_rope", torch.bfloat16, rows * H * d.d_rope),
        ctypes.byref(cache),
        _dev(seq_lens, "seq_lens", torch.int32, batch), max_seq_len,
        _dev(w_uk, "w_uk", torch.bfloat16, H * d.d_nope * d.d_latent),
        _dev(w_uv, "w_uv", torch.bfloat16, H * d.d_v * d.d_latent),
        float(sm_scale),
        _dev(out, "out", torch.bfloat16, rows * H * d.d_v),
        _dev(lse, "lse", torch.float32, rows * H),
        _dev(workspace, "workspace"), ws_bytes, _stream(stream))
    _check(st, "mla_prefill")


def mla_read_probe(buf, sink, stream=None):
    """One streaming read of the whole device tensor `buf` (a measurement
    helper: time it to get the read bandwidth this device achieves)."""
    nbytes = buf.numel() * buf.element_size()
    st = lib().mla_read_probe(_dev(buf, "buf"), nbytes, _dev(sink, "sink"), _stream(stream))
    _check(st, "mla_read_probe")


def mla_combine(dims, batch, num_splits, o_part, part_dtype, lse_part, out, lse, out_dtype,
                stream=None):
    d = dims_of(dims)
    H = d.num_heads
    st = lib().mla_combine(
        ctypes.byref(d), batch, num_splits,
        _dev(o_part, "o_part", _TORCH_DTYPE.get(part_dtype), batch * num_splits * H * d.d_latent),
        part_dtype,
        _dev(lse_part, "lse_part", torch.float32, batch * num_splits * H),
        _dev(out, "out", _TORCH_DTYPE.get(out_dtype), batch * H * d.d_latent),
        _dev(lse, "lse", torch.float32, batch * H),
        out_dtype, _stream(stream))
    _check(st, "mla_combine")


def mla_out_proj(dims, batch, o_lat, o_dtype, w_uv, w_dtype, out, out_dtype, stream=None):
    d = dims_of(dims)
    H = d.num_heads
    st = lib().mla_out_proj(
        ctypes.byref(d), batch,
        _dev(o_lat, "o_lat", _TORCH_DTYPE.get(o_dtype), batch * H * d.d_latent), o_dtype,
        _dev(w_uv, "w_uv", _TORCH_DTYPE.get(w_dtype), H * d.d_v * d.d_latent), w_dtype,
        _dev(out, "out", _TORCH_DTYPE.get(out_dtype), batch * H * d.d_v), out_dtype,
        _stream(stream))
    _check(st, "mla_out_proj")


def mla_combine_out_proj(dims, batch, num_splits, o_part, part_dtype, lse_part, w_uv, w_dtype, out,
                         out_dtype, lse, stream=None):
    d = dims_of(dims)
    H = d.num_heads
    st = lib().mla_combine_out_proj(
        ctypes.byref(d), batch, num_splits,
        _dev(o_part, "o_part", _TORCH_DTYPE.get(part_dtype), batch * num_splits * H * d.d_latent),
        part_dtype,
        _dev(lse_part, "lse_part", torch.float32, batch * num_splits * H),
        _dev(w_uv, "w_uv", _TORCH_DTYPE.get(w_dtype), H * d.d_v * d.d_latent), w_dtype,
        _dev(out, "out", _TORCH_DTYPE.get(out_dtype), batch * H * d.d_v), out_dtype,
        _dev(lse, "lse", torch.float32, batch * H),
        _stream(stream))
    _check(st, "mla_combine_out_proj")


def mla_o_proj_workspace(dims, batch, hidden):
    """Bytes of fp32 workspace mla_o_proj needs (0 for the tiny shape)."""
    d = dims_of(dims)
    return int(lib().mla_o_proj_workspace(ctypes.byref(d), batch, hidden))


def mla_o_proj(dims, batch, hidden, o, w_o, dtype, out, out_dtype, workspace=None, stream=None):
    """u[b] = W_O [o[b, 0]; ...; o[b, H-1]] into out [B, hidden]."""
    d = dims_of(dims)
    k = d.num_heads * d.d_v
    t = _TORCH_DTYPE.get(dtype)
    st = lib().mla_o_proj(ctypes.byref(d), batch, hidden, _dev(o, "o", t, batch * k),
                          _dev(w_o, "w_o", t, hidden * k), dtype,
                          _dev(out, "out", _TORCH_DTYPE.get(out_dtype), batch * hidden), out_dtype,
                          _dev(workspace, "workspace"),
                          workspace.numel() * workspace.element_size() if workspace is not None else 0,
                          _stream(stream))
    _check(st, "mla_o_proj")


def mla_cache_append_workspace(dims, batch, hidden):
    """Bytes of fp32 workspace mla_cache_append needs."""
    d = dims_of(dims)
    return int(lib().mla_cache_append_workspace(ctypes.byref(d), batch, hidden))


def mla_cache_append(dims, batch, hidden, h, w_dkv, w_kr, norm_gain, dtype, rms_eps, rope,
                     positions, cache, workspace, stream=None):
    """Write the cache entry (RMS-normed latent, rotated key) of one new token
    per sequence at row positions[b] of `cache`. `rope`: a Rope, or a number
    (plain RoPE with that base)."""
    d = dims_of(dims)
    t = _TORCH_DTYPE.get(dtype)
    st = lib().mla_cache_append(
        ctypes.byref(d), batch, hidden,
        _dev(h, "h", t, batch * hidden),
        _dev(w_dkv, "w_dkv", t, d.d_latent * hidden),
        _dev(w_kr, "w_kr", t, d.d_rope * hidden),
        _dev(norm_gain, "norm_gain", t, d.d_latent),
        dtype, float(rms_eps), ctypes.byref(rope_params(rope)),
        _dev(positions, "positions", torch.int32, batch),
        ctypes.byref(cache),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream))
    _check(st, "mla_cache_append")


def mla_cache_append_noalloc(dims, batch, hidden, h, w_dkv, w_kr, norm_gain, dtype, rms_eps, rope,
                             positions, cache, stream=None):
    """mla_cache_append with the library's own per-GPU scratch in place of a
    workspace (the call allocates nothing; calls on one GPU must not overlap)."""
    d = dims_of(dims)
    t = _TORCH_DTYPE.get(dtype)
    st = lib().mla_cache_append_noalloc(
        ctypes.byref(d), batch, hidden,
        _dev(h, "h", t, batch * hidden),
        _dev(w_dkv, "w_dkv", t, d.d_latent * hidden),
        _dev(w_kr, "w_kr", t, d.d_rope * hidden),
        _dev(norm_gain, "norm_gain", t, d.d_latent),
        dtype, float(rms_eps), ctypes.byref(rope_params(rope)),
        _dev(positions, "positions", torch.int32, batch),
        ctypes.byref(cache), _stream(stream))
    _check(st, "mla_cache_append_noalloc")


def mla_query_proj_workspace(dims, batch, hidden, d_qlatent):
    """Bytes of workspace mla_query_proj needs."""
    d = dims_of(dims)
    return int(lib().mla_query_proj_workspace(ctypes.byref(d), batch, hidden, d_qlatent))


def mla_query_proj(dims, batch, hidden, d_qlatent, h, w_dq, q_norm_gain, w_uq, w_qr, dtype, rms_eps, rope,
                   positions, q_nope, q_rope, workspace, stream=None):
    """q_nope [B, H, d_nope] and rotated q_rope [B, H, d_rope] of one new token
    per sequence from its hidden state (c_Q = RMSNorm(W_DQ h))."""
    d = dims_of(dims)
    t = _TORCH_DTYPE.get(dtype)
    H = d.num_heads
    st = lib().mla_query_proj(
        ctypes.byref(d), batch, hidden, d_qlatent,
        _dev(h, "h", t, batch * hidden),
        _dev(w_dq, "w_dq", t, d_qlatent * hidden),
        _dev(q_norm_gain, "q_norm_gain", t, d_qlatent),
        _dev(w_uq, "w_uq", t, H * d.d_nope * d_qlatent),
        _dev(w_qr, "w_qr", t, H * d.d_rope * d_qlatent),
        dtype, float(rms_eps), ctypes.byref(rope_params(rope)),
        _dev(positions, "positions", torch.int32, batch),
        _dev(q_nope, "q_nope", t, batch * H * d.d_nope),
        _dev(q_rope, "q_rope", t, batch * H * d.d_rope),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream))
    _check(st, "mla_query_proj")


def mla_split_chunk(max_seq_len, num_splits):
    return lib().mla_split_chunk(max_seq_len, num_splits)


def mla_suggest_splits(batch, max_seq_len, total_tokens, num_cus):
    return lib().mla_suggest_splits(batch, max_seq_len, total_tokens, num_cus)


def mla_time_next_launch(start, stop):
    """The library's next kernel launch from this thread records `start` and
    `stop` around its own execution: raw hipEvent_t handles (int), or
    torch.cuda.Event objects made with enable_timing=True, or None. A torch
    event must exist already: record it once before handing it over."""
    def handle(e):
        if e is None:
            return None
        if isinstance(e, int):
            return ctypes.c_void_p(e)
        if not e.cuda_event:
            raise ValueError("record the event once before passing it (torch creates events lazily)")
        return ctypes.c_void_p(e.cuda_event)
    return lib().mla_time_next_launch(handle(start), handle(stop))


def status_string(status):
    return lib().mla_status_string(status).decode()


def last_hip_error():
    return lib().mla_last_hip_error()
