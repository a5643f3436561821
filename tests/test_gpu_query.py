"""GPU parity of the query path (mla_query_proj) against the float64 oracle,
and of the whole layer chain from a new token's hidden state to the
attention output u = W_O [o_1; ...; o_H]:

  h -> mla_query_proj -> mla_absorb_q -> mla_decode -> (merge +) W_UV -> mla_o_proj

against oracle.query_path -> oracle.decode (non-absorbed) ->
oracle.output_projection on the same seeded inputs.

Bounds: relative L2 <= 1e-2 (bf16 with fp32 accumulation; the kernels round
c_Q and the outputs to bf16, about 2e-3 relative each) and max abs within
3e-2 of the largest reference value for the query; the chain is held to the
decode's own bounds (relative L2 <= 1e-2, max abs <= 3e-2).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from mla_synth import DSV2, make_inputs, make_oproj_inputs, make_query_inputs, oracle_args

pytestmark = pytest.mark.gpu

YARN = dict(yarn_scale=40.0, yarn_alpha=1.0, yarn_beta=32.0, orig_ctx=4096)   # the pages' YaRN parameters


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_28_amd as mla
    mla.lib()     # fails loudly when the library is missing


def _rel(x, y):
    return float(np.linalg.norm((x - y).ravel()) / np.linalg.norm(y.ravel()))


def _rope(mla, yarn):
    if yarn:
        return mla.Rope(10000.0, YARN["yarn_scale"], YARN["yarn_alpha"], YARN["yarn_beta"], YARN["orig_ctx"])
    return mla.Rope(10000.0, 1.0, 1.0, 32.0, 4096)


def _freqs(yarn):
    return oracle.rope_frequencies(DSV2.d_rope, 10000.0, **(YARN if yarn else {}))


def _gpu_query(inp, yarn):
    import mla_latent_kv_28_amd as mla
    d, B = inp.dims, inp.h.shape[0]
    dev = "cuda"
    qn = torch.empty((B, d.num_heads, d.d_nope), dtype=torch.bfloat16, device=dev)
    qr = torch.empty((B, d.num_heads, d.d_rope), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(mla.mla_query_proj_workspace(d, B, d.hidden, inp.d_qlatent), dtype=torch.uint8, device=dev)
    print("case: query B=%d yarn=%s positions=%s" % (B, yarn, inp.positions[:6].tolist()), flush=True)
    mla.mla_query_proj(d, B, d.hidden, inp.d_qlatent, inp.h.to(dev), inp.w_dq.to(dev),
                       None if inp.gain is None else inp.gain.to(dev), inp.w_uq.to(dev), inp.w_qr.to(dev),
                       mla.BF16, inp.eps, _rope(mla, yarn), torch.from_numpy(inp.positions).to(dev), qn, qr, ws)
    torch.cuda.synchronize()
    return qn, qr


def _oracle_query(inp, yarn):
    f = lambda t: None if t is None else t.double().numpy()
    return oracle.query_path(f(inp.h), f(inp.w_dq), f(inp.w_uq), f(inp.w_qr), inp.positions, inp.eps,
                             _freqs(yarn), inp.dims.num_heads, f(inp.gain))


def _check(got, ref, rel=1e-2, absb=3e-2):
    r = _rel(got, ref)
    m = float(np.abs(got - ref).max())
    print("rel_l2 %.3e max_abs %.3e (max|ref| %.3e)" % (r, m, float(np.abs(ref).max())), flush=True)
    assert np.all(np.isfinite(got))
    assert r <= rel
    assert m <= absb


@pytest.mark.parametrize("B,yarn,gain", [(32, False, False), (32, True, True), (45, True, False), (1, False, True)])
def test_query_path_against_oracle(B, yarn, gain):
    # 45 rows: a second, ragged 32-row block; positions up to the 160K YaRN range
    inp = make_query_inputs(DSV2, batch=B, seed=B, max_position=163840 if yarn else 4096, with_gain=gain)
    qn, qr = _gpu_query(inp, yarn)
    _, ref_n, ref_r = _oracle_query(inp, yarn)
    _check(qn.double().cpu().numpy(), ref_n, absb=3e-2 * np.abs(ref_n).max())
    _check(qr.double().cpu().numpy(), ref_r, absb=3e-2 * np.abs(ref_r).max())


def test_query_path_contraction_tails():
    # a hidden size that is not a multiple of the W_DQ product's 1024-wide
    # contraction parts, and a d'_c whose quarter is not a multiple of the
    # second product's 192-wide wave steps: both products take the instances
    # that zero the operands past the contraction's end
    import dataclasses
    d = dataclasses.replace(DSV2, hidden=4144)
    inp = make_query_inputs(d, batch=37, seed=9, d_qlatent=1280, with_gain=True)
    qn, qr = _gpu_query(inp, False)
    _, ref_n, ref_r = _oracle_query(inp, False)
    _check(qn.double().cpu().numpy(), ref_n, absb=3e-2 * np.abs(ref_n).max())
    _check(qr.double().cpu().numpy(), ref_r, absb=3e-2 * np.abs(ref_r).max())


def test_query_rotation_positions_zero_and_wrap():
    # position 0 leaves the rotary query unrotated: equal to the same inputs
    # with YaRN frequencies (frequencies do not matter at 0); a large position
    # turns the fastest pair by p rad, taken modulo 2 pi in double precision
    inp = make_query_inputs(DSV2, batch=4, seed=5, positions=[0, 0, 1 << 20, (1 << 31) - 1])
    qn0, qr0 = _gpu_query(inp, False)
    qn1, qr1 = _gpu_query(inp, True)
    assert torch.equal(qn0, qn1)
    assert torch.equal(qr0[:2], qr1[:2])
    _, _, ref_r = _oracle_query(inp, False)
    _check(qr0.double().cpu().numpy(), ref_r, absb=3e-2 * np.abs(ref_r).max())


def test_layer_chain_from_hidden_state_to_attention_output():
    # h -> query path -> absorb -> decode (3 splits) -> merge + W_UV -> W_O,
    # against the oracle's query path, non-absorbed decode and output projection
    import mla_latent_kv_28_amd as mla
    from mla_latent_kv_28_amd.pipeline import DecodePipeline
    lens = [900, 33, 2048, 1]
    B = len(lens)
    cache_inp = make_inputs("dsv2_b32_l4096", seq_lens=lens, pad_fill=float("nan"))
    q_inp = make_query_inputs(DSV2, batch=B, seed=9, positions=[L - 1 for L in lens], with_gain=True)
    qn, qr = _gpu_query(q_inp, True)
    _, ref_qn, ref_qr = _oracle_query(q_inp, True)
    # GPU side: the query path's bf16 outputs feed the pipeline
    cache_inp.q_nope, cache_inp.q_rope = qn.cpu(), qr.cpu()
    pipe = DecodePipeline(cache_inp, num_splits=3)
    o, _ = pipe.run()
    _, w_o = make_oproj_inputs(DSV2, B, seed=4)
    w_o = w_o.cuda()
    u = torch.empty((B, DSV2.hidden), dtype=torch.float32, device="cuda")
    work = torch.empty(mla.mla_o_proj_workspace(DSV2, B, DSV2.hidden) // 4, dtype=torch.float32, device="cuda")
    mla.mla_o_proj(DSV2, B, DSV2.hidden, o, w_o, mla.BF16, u, mla.F32, work)
    torch.cuda.synchronize()
    # oracle side: the float64 query (not the GPU's bf16 one) all the way through
    a = oracle_args(cache_inp)
    a["q_nope"], a["q_rope"] = ref_qn, ref_qr
    ref_o, _ = oracle.decode(**a)
    ref_u = oracle.output_projection(ref_o, w_o.double().cpu().numpy())
    print("chain: per-head outputs", flush=True)
    _check(o.double().cpu().numpy(), ref_o)
    print("chain: attention output u", flush=True)
    _check(u.double().cpu().numpy(), ref_u)
