"""One MLA decode step through libmla: absorb -> decode -> combine -> out-proj.

Holds the device tensors of one workload and enqueues the four C-ABI calls on
the current stream. Allocation happens once, in the constructor.
"""

import torch

from . import (BF16, F32, FP8_E4M3, kv_cache, mla_absorb_q, mla_combine, mla_combine_out_proj,
               mla_decode, mla_decode_multi, mla_out_proj, mla_suggest_splits)

NUM_CUS = 256


class DecodePipeline:
    """Device copy of a workload plus the buffers of the decode step.

    `inp` is any object with the fields of mla_synth.Inputs (dims, dtype,
    seq_lens, sm_scale, q_nope, q_rope, w_uk, w_uv, rows or codes/scale/rope,
    layout, seq_stride, page_size, block_table).
    o_lat_dtype: precision of the merged latent output handed to out-proj, and
                 of the split partials when there is more than one split.
    out_dtype:   precision of the final per-head output.
    fuse:        with several splits of bf16 partials at the DeepSeek-V2 shape,
                 run merge and out-proj as one call (mla_combine_out_proj; o_lat
                 is then not written).
    tokens_per_seq: n new tokens per sequence scored together, causally
                 (mla_decode_multi); q_nope / q_rope then hold batch * n rows,
                 row b n + t for token t, and so do the outputs.
    """

    def __init__(self, inp, num_splits=None, o_lat_dtype=None, out_dtype=None, device="cuda",
                 fuse=True, tokens_per_seq=None):
        d = inp.dims
        self.dims = d
        self.seqs = inp.batch
        self.tokens_per_seq = int(getattr(inp, "tokens_per_seq", 1) if tokens_per_seq is None else tokens_per_seq)
        self.batch = inp.batch * self.tokens_per_seq     # query rows
        if inp.q_nope.shape[0] != self.batch or inp.q_rope.shape[0] != self.batch:
            raise ValueError("queries hold %d rows, expected %d sequences x %d tokens"
                             % (inp.q_nope.shape[0], inp.batch, self.tokens_per_seq))
        self.max_seq_len = inp.max_seq_len
        self.sm_scale = inp.sm_scale
        self.compute = F32 if inp.dtype == "f32" else BF16
        self.o_lat_dtype = self.compute if o_lat_dtype is None else o_lat_dtype
        self.out_dtype = self.compute if out_dtype is None else out_dtype
        dev = torch.device(device)
        self.q_nope = inp.q_nope.to(dev).contiguous()
        self.q_rope = inp.q_rope.to(dev).contiguous()
        self.w_uk = inp.w_uk.to(dev).contiguous()
        self.w_uv = inp.w_uv.to(dev).contiguous()
        self.seq_lens = torch.from_numpy(inp.seq_lens).to(dev)
        bt = None
        if inp.layout == "paged":
            bt = torch.from_numpy(inp.block_table).to(dev).contiguous()
        self.block_table = bt
        paged = dict(page_size=inp.page_size, block_table=bt,
                     max_pages_per_seq=0 if bt is None else bt.shape[1],
                     seq_stride=inp.seq_stride)
        if inp.dtype == "fp8":
            self.codes = inp.codes.to(dev).contiguous()
            self.rope = inp.rope.to(dev).contiguous()
            self.scale = inp.scale.to(dev).contiguous()
            self.cache = kv_cache(FP8_E4M3, self.codes, rope=self.rope, scale=self.scale,
                                  row_stride=d.d_latent, rope_stride=d.d_rope, **paged)
        else:
            self.rows = inp.rows.to(dev).contiguous()
            self.cache = kv_cache(self.compute, self.rows, row_stride=d.width, **paged)

        if num_splits is None:
            num_splits = inp.splits or mla_suggest_splits(
                self.batch, self.max_seq_len,
                int(inp.seq_lens.astype("int64").sum()) * self.tokens_per_seq, NUM_CUS)
        self.num_splits = int(num_splits)
        B, H, S = self.batch, d.num_heads, self.num_splits
        cdt = torch.float32 if self.compute == F32 else torch.bfloat16
        odt = torch.float32 if self.o_lat_dtype == F32 else torch.bfloat16
        fdt = torch.float32 if self.out_dtype == F32 else torch.bfloat16
        self.q_lat = torch.empty((B, H, d.width), dtype=cdt, device=dev)
        if S > 1:
            self.o_part = torch.empty((B, S, H, d.d_latent), dtype=odt, device=dev)
            self.lse_part = torch.empty((B, S, H), dtype=torch.float32, device=dev)
        else:
            self.o_part = self.lse_part = None
        self.o_lat = torch.empty((B, H, d.d_latent), dtype=odt, device=dev)
        self.fused = (fuse and 1 < S <= 64 and self.o_lat_dtype == BF16 and self.compute == BF16
                      and (d.num_heads, d.d_latent, d.d_rope, d.d_nope, d.d_v) == (128, 512, 64, 128, 128))
        self.lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        self.out = torch.empty((B, H, d.d_v), dtype=fdt, device=dev)

    def absorb(self, stream=None):
        mla_absorb_q(self.dims, self.batch, self.q_nope, self.q_rope, self.w_uk, self.q_lat,
                     self.compute, stream)

    def decode(self, stream=None):
        split = self.num_splits > 1
        out = self.o_part if split else self.o_lat
        lse = self.lse_part if split else self.lse
        if self.tokens_per_seq > 1:
            mla_decode_multi(self.dims, self.seqs, self.tokens_per_seq, self.q_lat, self.cache, self.seq_lens,
                             self.max_seq_len, self.sm_scale, self.num_splits, out, lse, self.o_lat_dtype,
                             stream)
        else:
            mla_decode(self.dims, self.batch, self.q_lat, self.cache, self.seq_lens,
                       self.max_seq_len, self.sm_scale, self.num_splits, out, lse,
                       self.o_lat_dtype, stream)

    def combine(self, stream=None):
        if self.num_splits > 1:
            mla_combine(self.dims, self.batch, self.num_splits, self.o_part, self.o_lat_dtype,
                        self.lse_part, self.o_lat, self.lse, self.o_lat_dtype, stream)

    def out_proj(self, stream=None):
        mla_out_proj(self.dims, self.batch, self.o_lat, self.o_lat_dtype, self.w_uv,
                     self.compute, self.out, self.out_dtype, stream)

    def combine_out_proj(self, stream=None):
        mla_combine_out_proj(self.dims, self.batch, self.num_splits, self.o_part, self.o_lat_dtype,
                             self.lse_part, self.w_uv, self.compute, self.out, self.out_dtype, self.lse,
                             stream)

    def run(self, stream=None):
        self.absorb(stream)
        self.decode(stream)
        if self.fused:
            self.combine_out_proj(stream)
        else:
            self.combine(stream)
            self.out_proj(stream)
        return self.out, self.lse
