"""The library's calls inside HIP graphs: each call sequence is captured once,
replayed several times with the program's own eager work and
synchronisations between the replays, and every replay is held bit for bit
to the same calls run eagerly (the benchmark times the decode step this
way). No call of the library records a memset or allocates, so captured
calls replay the eager arithmetic exactly.
"""

import pytest
import torch

from mla_synth import DSV2, make_append_inputs, make_inputs, make_query_inputs

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_28_amd as mla
    mla.lib()     # fails loudly when the library is missing


def _replay_equals_eager(run, outputs, clobber):
    """run(): enqueue the calls on the current stream; outputs: tensors they
    write; clobber(): eager work that overwrites the outputs in between."""
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        run()
    for i in range(REPLAYS):
        clobber()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(outputs, eager):
            assert torch.equal(t, e), "replay %d differs from the eager result" % i
        # eager work on the same tensors between replays
        with torch.cuda.stream(stream):
            run()
        torch.cuda.synchronize()


@pytest.mark.parametrize("splits", [1, 8])
def test_decode_step_in_a_graph(splits):
    from mla_latent_kv_28_amd.pipeline import DecodePipeline
    inp = make_inputs("dsv2_b32_l4096", seq_lens=[1000, 77, 4096, 1, 513, 32], pad_fill=float("nan"))
    pipe = DecodePipeline(inp, num_splits=splits)
    print("case: graph decode step splits=%d fused=%s" % (splits, pipe.fused), flush=True)
    outs = [pipe.out, pipe.lse, pipe.q_lat]

    def clobber():
        for t in outs:
            t.fill_(7.0)

    _replay_equals_eager(pipe.run, outs, clobber)


def test_multi_token_decode_in_a_graph():
    from mla_latent_kv_28_amd.pipeline import DecodePipeline
    inp = make_inputs("dsv2_b32_l4096", seq_lens=[300, 2, 700], pad_fill=float("nan"), tokens_per_seq=3)
    pipe = DecodePipeline(inp, num_splits=2)
    print("case: graph multi-token decode", flush=True)
    outs = [pipe.out, pipe.lse]
    _replay_equals_eager(pipe.run, outs, lambda: [t.fill_(-3.0) for t in outs])


def test_query_append_and_prefill_in_a_graph():
    import mla_latent_kv_28_amd as mla
    d, dev = DSV2, "cuda"
    B = 4
    # query path
    q = make_query_inputs(d, batch=B, seed=2, max_position=163840, with_gain=True)
    qn = torch.empty((B, d.num_heads, d.d_nope), dtype=torch.bfloat16, device=dev)
    qr = torch.empty((B, d.num_heads, d.d_rope), dtype=torch.bfloat16, device=dev)
    qws = torch.empty(mla.mla_query_proj_workspace(d, B, d.hidden, q.d_qlatent), dtype=torch.uint8, device=dev)
    qargs = [t.to(dev) for t in (q.h, q.w_dq, q.gain, q.w_uq, q.w_qr)]
    qpos = torch.from_numpy(q.positions).to(dev)
    rope = mla.Rope(10000.0, 40.0, 1.0, 32.0, 4096)
    # cache append into a contiguous bf16 cache
    a = make_append_inputs(d, batch=B, seed=3, max_position=64)
    rows = torch.zeros((B * 64, d.width), dtype=torch.bfloat16, device=dev)
    cache = mla.kv_cache(mla.BF16, rows, row_stride=d.width, seq_stride=64)
    aws = torch.empty(mla.mla_cache_append_workspace(d, B, d.hidden), dtype=torch.uint8, device=dev)
    aargs = [t.to(dev) for t in (a.h, a.w_dkv, a.w_kr)]
    apos = torch.from_numpy(a.positions).to(dev)
    # prefill over a separate cache
    pinp = make_inputs("dsv2_b32_l4096", seq_lens=[200, 77], tokens_per_seq=77)
    prow = pinp.rows.to(dev)
    pcache = mla.kv_cache(mla.BF16, prow, row_stride=d.width, seq_stride=pinp.seq_stride)
    plens = torch.from_numpy(pinp.seq_lens).to(dev)
    pq = [pinp.q_nope.to(dev), pinp.q_rope.to(dev)]
    pw = [pinp.w_uk.to(dev), pinp.w_uv.to(dev)]
    pout = torch.empty((2 * 77, d.num_heads, d.d_v), dtype=torch.bfloat16, device=dev)
    plse = torch.empty((2 * 77, d.num_heads), dtype=torch.float32, device=dev)
    pws = torch.empty(mla.mla_prefill_workspace(d, 2, pinp.max_seq_len), dtype=torch.uint8, device=dev)
    print("case: graph query path + cache append + prefill", flush=True)

    def run():
        mla.mla_query_proj(d, B, d.hidden, q.d_qlatent, qargs[0], qargs[1], qargs[2], qargs[3], qargs[4], mla.BF16,
                           q.eps, rope, qpos, qn, qr, qws)
        mla.mla_cache_append(d, B, d.hidden, aargs[0], aargs[1], aargs[2], None, mla.BF16, a.eps, rope, apos,
                             cache, aws)
        mla.mla_prefill(d, 2, 77, pq[0], pq[1], pcache, plens, pinp.max_seq_len, pw[0], pw[1], pinp.sm_scale,
                        pout, plse, pws)

    outs = [qn, qr, rows, pout, plse]

    def clobber():
        qn.fill_(1.0)
        qr.fill_(1.0)
        rows.fill_(0.0)
        pout.fill_(2.0)
        plse.fill_(2.0)

    _replay_equals_eager(run, outs, clobber)
