"""GPU parity of the prefill (mla_prefill: n new tokens per sequence in the
non-absorbed form, causal) against oracle.prefill, and against the absorbed
path (absorb -> mla_decode_multi -> merge -> W_UV) on the same inputs.

Bounds: the decode's bf16 bounds, relative L2 <= 1e-2 and max abs <= 3e-2
(bf16 operands with fp32 accumulation; the kernels also round the keys and
values k^C, v^C to bf16 once, relative 2^-9). The two GPU paths are held to
each other at twice that relative bound.
"""

import numpy as np
import pytest
import torch

import oracle
from mla_synth import make_inputs, oracle_args

pytestmark = pytest.mark.gpu

BF16_REL, BF16_ABS = 1e-2, 3e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_28_amd as mla
    mla.lib()     # fails loudly when the library is missing


def _rel(x, y):
    den = np.linalg.norm(y.ravel())
    return float(np.linalg.norm((x - y).ravel()) / (den if den > 0 else 1.0))


def _check(out, ref, rel, absb=None):
    assert np.all(np.isfinite(out))
    r = _rel(out, ref)
    m = float(np.abs(out - ref).max()) if out.size else 0.0
    print("rel_l2 %.3e max_abs %.3e (max|ref| %.3e)" % (r, m, float(np.abs(ref).max())), flush=True)
    assert r <= rel
    if absb is not None:
        assert m <= absb


def _lse_check(lse, ref_lse, tol=2e-2):
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.all(lse[~fin] == -np.inf)
    if fin.any():
        d = np.abs(lse[fin] - ref_lse[fin])
        print("lse max abs err %.3e" % d.max(), flush=True)
        assert np.all(d <= tol + 4e-3 * np.abs(ref_lse[fin]))


def _prefill(inp, n):
    import mla_latent_kv_28_amd as mla
    d = inp.dims
    B, L = inp.batch, inp.max_seq_len
    print("case: prefill n=%d B=%d lens=%s layout=%s page=%d" % (n, B, inp.seq_lens[:8].tolist(), inp.layout,
                                                                  inp.page_size), flush=True)
    dev = "cuda"
    rows = inp.rows.to(dev)
    bt = None if inp.block_table is None else torch.from_numpy(inp.block_table).to(dev).contiguous()
    cache = mla.kv_cache(mla.BF16, rows, row_stride=d.width, page_size=inp.page_size, seq_stride=inp.seq_stride,
                         block_table=bt, max_pages_per_seq=0 if bt is None else bt.shape[1])
    out = torch.empty((B * n, d.num_heads, d.d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B * n, d.num_heads), dtype=torch.float32, device=dev)
    ws = torch.empty(max(mla.mla_prefill_workspace(d, B, L), 16), dtype=torch.uint8, device=dev)
    mla.mla_prefill(d, B, n, inp.q_nope.to(dev), inp.q_rope.to(dev), cache, torch.from_numpy(inp.seq_lens).to(dev),
                    L, inp.w_uk.to(dev), inp.w_uv.to(dev), inp.sm_scale, out, lse, ws)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy()


CASES = {
    # name: (lens, n, layout overrides)
    "whole_prompts_300": ([300, 300], 300, {}),                    # 3 query blocks, the last ragged
    "chunk_after_prefix": ([700, 129, 1000], 129, {}),            # new tokens after cached ones
    "shorter_than_n": ([50, 5, 64], 64, {}),                      # early tokens see no row
    "paged64": ([300, 77], 77, dict(layout="paged", page_size=64)),
    "paged16": ([200, 33], 33, dict(layout="paged", page_size=16)),
    "one_token": ([1, 40], 1, {}),                                 # a decode in the non-absorbed form
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_prefill_against_oracle(case):
    lens, n, over = CASES[case]
    inp = make_inputs("dsv2_b32_l4096", seq_lens=lens, pad_fill=float("nan"), tokens_per_seq=n, **over)
    out, lse = _prefill(inp, n)
    ref, ref_lse = oracle.prefill(n=n, **oracle_args(inp))
    _check(out, ref, BF16_REL, BF16_ABS)
    _lse_check(lse, ref_lse)


@pytest.mark.parametrize("factor", [-1.0, 0.0])
def test_prefill_non_positive_scale(factor):
    # the kernel instance for scales <= 0 (scores scaled before the maximum):
    # a negated scale reverses the ranking of the keys, zero makes every
    # visible key weigh the same
    import dataclasses
    lens, n = [300, 129], 129
    inp = make_inputs("dsv2_b32_l4096", seq_lens=lens, pad_fill=float("nan"), tokens_per_seq=n)
    inp = dataclasses.replace(inp, sm_scale=factor * inp.sm_scale)
    out, lse = _prefill(inp, n)
    ref, ref_lse = oracle.prefill(n=n, **oracle_args(inp))
    _check(out, ref, BF16_REL, BF16_ABS)
    _lse_check(lse, ref_lse)


def test_prefill_matches_the_absorbed_multi_token_path():
    from mla_latent_kv_28_amd.pipeline import DecodePipeline
    lens, n = [700, 129, 1000], 129
    inp = make_inputs("dsv2_b32_l4096", seq_lens=lens, tokens_per_seq=n)
    out, lse = _prefill(inp, n)
    pipe = DecodePipeline(inp, num_splits=2)
    o_abs, l_abs = pipe.run()
    torch.cuda.synchronize()
    _check(out, o_abs.double().cpu().numpy(), 2 * BF16_REL)
    _lse_check(lse, l_abs.double().cpu().numpy())


def test_prefill_full_prompt_4096_sampled():
    # one 4096-token prompt (32 query blocks, 64 key blocks for the last):
    # sampled (token, head) outputs against the oracle's decode of each
    # token's causal prefix with its own query
    n = 4096
    inp = make_inputs("dsv2_b32_l4096", batch=1, tokens_per_seq=n)
    out, lse = _prefill(inp, n)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    a = oracle_args(inp)
    got, ref, gl, rl = [], [], [], []
    for t in [0, 1, 63, 64, 127, 128, 1000, 2047, 4095]:
        heads = [32 * w + (3 * t + 7 * w) % 32 for w in range(4)]
        q_n, q_r = a["q_nope"][t:t + 1], a["q_rope"][t:t + 1]
        lens = np.array([t + 1], dtype=np.int32)
        ro, rlse = oracle.decode_heads(q_n, q_r, a["w_uk"], a["w_uv"], a["cache"], lens, a["sm_scale"], 0, heads)
        got.append(out[t, heads])
        ref.append(ro)
        gl.append(lse[t, heads])
        rl.append(rlse)
    print("checked %d (token, head) outputs" % sum(len(g) for g in got), flush=True)
    _check(np.concatenate(got), np.concatenate(ref), BF16_REL, BF16_ABS)
    _lse_check(np.concatenate(gl), np.concatenate(rl))
