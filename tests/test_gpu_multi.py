"""GPU parity of the decode of several new tokens per sequence
(mla_decode_multi; the DeepSeek-V3 blog, section 3 on multi-token prediction)
against oracle.decode_multi: token t of sequence b attends, causally, to cache
rows 0 .. L_b - n + t.

Every case runs absorb -> mla_decode_multi -> merge -> W_UV on the GPU and the
float64 non-absorbed oracle on the host, with the decode's own bounds
(relative L2 <= 1e-2, max abs <= 3e-2 for bf16; fp8 against the dequantised
cache likewise). At full size, where the oracle checks a sample, every query
row is also held bit for bit to mla_decode over a cache in which each row has
its own copy of its sequence: the one-token decode of that row's causal
prefix, whose own parity is tested elsewhere.
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


def _run(inp, **kw):
    from mla_latent_kv_28_amd.pipeline import DecodePipeline
    print("case: %s n=%d B=%d lens=%s layout=%s splits=%s" % (inp.name, inp.tokens_per_seq, inp.batch,
                                                               inp.seq_lens[:8].tolist(), inp.layout,
                                                               kw.get("num_splits")), flush=True)
    pipe = DecodePipeline(inp, **kw)
    out, lse = pipe.run()
    torch.cuda.synchronize()
    return pipe, out.double().cpu().numpy(), lse.double().cpu().numpy()


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


def _visible(lens, n):
    """Rows each query row attends to: L_b - n + t + 1, at least 0."""
    return np.array([max(0, int(L) - n + 1 + t) for L in lens for t in range(n)], dtype=np.int32)


RAGGED = [1, 2, 77, 1000, 33, 513]     # the first two are shorter than n: their early tokens see nothing


@pytest.mark.parametrize("n,splits", [(2, 1), (3, 3), (4, 8)])
def test_multi_bf16_contiguous_ragged(n, splits):
    inp = make_inputs("dsv2_b32_l4096", seq_lens=RAGGED, pad_fill=float("nan"), tokens_per_seq=n)
    _, out, lse = _run(inp, num_splits=splits)
    ref, ref_lse = oracle.decode_multi(n=n, **oracle_args(inp))
    empty = _visible(RAGGED, n) == 0
    assert empty.any() and np.all(out[empty] == 0)
    _check(out, ref, BF16_REL, BF16_ABS)
    _lse_check(lse, ref_lse)


def test_multi_paged_equals_contiguous_and_oracle():
    lens = [130, 64, 3, 700, 0, 191]
    common = dict(seq_lens=lens, pad_fill=float("nan"), tokens_per_seq=3)
    cont = make_inputs("dsv2_b32_l4096", **common)
    paged = make_inputs("dsv2_b32_l4096", layout="paged", page_size=64, **common)
    _, out_c, lse_c = _run(cont, num_splits=2)
    _, out_p, lse_p = _run(paged, num_splits=2)
    assert np.array_equal(out_c, out_p) and np.array_equal(lse_c, lse_p)
    ref, ref_lse = oracle.decode_multi(n=3, **oracle_args(paged))
    _check(out_p, ref, BF16_REL, BF16_ABS)
    _lse_check(lse_p, ref_lse)


@pytest.mark.parametrize("page_size", [16, 128])
def test_multi_paged_other_page_sizes(page_size):
    inp = make_inputs("dsv2_b32_l4096", seq_lens=[200, 33, 2], layout="paged", page_size=page_size,
                      pad_fill=float("nan"), tokens_per_seq=2)
    _, out, lse = _run(inp, num_splits=1)
    ref, ref_lse = oracle.decode_multi(n=2, **oracle_args(inp))
    _check(out, ref, BF16_REL, BF16_ABS)
    _lse_check(lse, ref_lse)


@pytest.mark.parametrize("splits", [1, 2])
def test_multi_fp8_cache(splits):
    inp = make_inputs("fp8_b128_l8192", seq_lens=[600, 97, 1], pad_fill=float("nan"), tokens_per_seq=2)
    _, out, lse = _run(inp, num_splits=splits)
    ref, ref_lse = oracle.decode_multi(n=2, **oracle_args(inp))
    _check(out, ref, BF16_REL, BF16_ABS)
    _lse_check(lse, ref_lse)


# --- against the one-token decode of each row's causal prefix, bit for bit --------

def _decode_rows(pipe, cache, lens_v):
    """mla_decode of the pipeline's absorbed queries (one per row) over `cache`
    with lengths lens_v; the same split count and output precision."""
    import mla_latent_kv_28_amd as mla
    R, H, D = pipe.batch, pipe.dims.num_heads, pipe.dims.d_latent
    S = pipe.num_splits
    odt = pipe.o_part.dtype if S > 1 else pipe.o_lat.dtype
    out = torch.empty((R, S, H, D) if S > 1 else (R, H, D), dtype=odt, device="cuda")
    lse = torch.empty((R, S, H) if S > 1 else (R, H), dtype=torch.float32, device="cuda")
    mla.mla_decode(pipe.dims, R, pipe.q_lat, cache, torch.from_numpy(lens_v).cuda(), pipe.max_seq_len,
                   pipe.sm_scale, S, out, lse, pipe.o_lat_dtype)
    torch.cuda.synchronize()
    return out, lse


def _multi_parts(pipe):
    pipe.absorb()
    pipe.decode()
    torch.cuda.synchronize()
    if pipe.num_splits > 1:
        return pipe.o_part.clone(), pipe.lse_part.clone()
    return pipe.o_lat.clone(), pipe.lse.clone()


def _sampled_oracle(inp, out, lse, rows, n):
    """out[bv, heads] against the oracle for a few query rows: row bv = b n + t
    is sequence b's decode with its own query over L_b - n + t + 1 rows."""
    a = oracle_args(inp)
    got, ref, gl, rl = [], [], [], []
    for bv in rows:
        b, t = divmod(bv, n)
        heads = [32 * w + (5 * bv + 13 * w) % 32 for w in range(4)]
        q_n, q_r = np.zeros_like(a["q_nope"][:inp.batch]), np.zeros_like(a["q_rope"][:inp.batch])
        q_n[b], q_r[b] = a["q_nope"][bv], a["q_rope"][bv]
        lens = inp.seq_lens.copy()
        lens[b] = max(0, int(lens[b]) - n + 1 + t)
        ro, rlse = oracle.decode_heads(q_n, q_r, a["w_uk"], a["w_uv"], a["cache"], lens, a["sm_scale"], b, heads)
        got.append(out[bv, heads])
        ref.append(ro)
        gl.append(lse[bv, heads])
        rl.append(rlse)
    print("checked %d (row, head) outputs" % sum(len(g) for g in got), flush=True)
    _check(np.concatenate(got), np.concatenate(ref), BF16_REL, BF16_ABS)
    _lse_check(np.concatenate(gl), np.concatenate(rl))


def test_multi_equals_decode_on_replicated_pages_longest_first():
    # 48 sequences x 4 tokens x 2 splits = 384 items: more than the compute
    # units, so the items are handed out longest first
    import mla_latent_kv_28_amd as mla
    from mla_latent_kv_28_amd.pipeline import DecodePipeline
    n, ps = 4, 64
    lens = np.random.default_rng(3).integers(1, 700, size=48)
    lens[:3] = [1, 3, 4]
    inp = make_inputs("dsv2_b32_l4096", seq_lens=lens.tolist(), layout="paged", page_size=ps,
                      pad_fill=float("nan"), tokens_per_seq=n)
    pipe = DecodePipeline(inp, num_splits=2)
    print("case: replicated pages n=%d B=%d splits=2" % (n, inp.batch), flush=True)
    o_m, l_m = _multi_parts(pipe)
    bt_v = torch.from_numpy(np.repeat(inp.block_table, n, axis=0)).cuda().contiguous()
    cache_v = mla.kv_cache(mla.BF16, pipe.rows, row_stride=pipe.dims.width, page_size=ps, block_table=bt_v,
                           max_pages_per_seq=bt_v.shape[1])
    o_d, l_d = _decode_rows(pipe, cache_v, _visible(lens, n))
    assert torch.equal(o_m, o_d) and torch.equal(l_m, l_d)
    out, lse = pipe.run()
    torch.cuda.synchronize()
    _sampled_oracle(inp, out.double().cpu().numpy(), lse.double().cpu().numpy(), [0, 1, 2, 3, 9, 50, 191], n)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_full_size_multi_two_tokens(dtype):
    # the 32-sequence, 4096-token workload with two new tokens per sequence (the
    # fp8 cache at the same size): every row bit for bit against mla_decode over
    # a cache holding a copy of its sequence per row, a sample against the oracle
    import mla_latent_kv_28_amd as mla
    from mla_latent_kv_28_amd.pipeline import DecodePipeline
    n = 2
    inp = make_inputs("dsv2_b32_l4096", dtype=dtype, tokens_per_seq=n)
    pipe = DecodePipeline(inp)
    print("case: full size %s n=%d B=%d splits=%d" % (dtype, n, inp.batch, pipe.num_splits), flush=True)
    o_m, l_m = _multi_parts(pipe)
    B, stride, d = inp.batch, inp.seq_stride, pipe.dims
    if dtype == "fp8":
        codes = pipe.codes.view(B, stride, -1).repeat_interleave(n, dim=0).reshape(B * n * stride, -1)
        rope = pipe.rope.view(B, stride, -1).repeat_interleave(n, dim=0).reshape(B * n * stride, -1)
        scale = pipe.scale.view(B, stride).repeat_interleave(n, dim=0).reshape(-1)
        cache_v = mla.kv_cache(mla.FP8_E4M3, codes.contiguous(), rope=rope.contiguous(), scale=scale.contiguous(),
                               row_stride=d.d_latent, rope_stride=d.d_rope, seq_stride=stride)
    else:
        rows = pipe.rows.view(B, stride, -1).repeat_interleave(n, dim=0).reshape(B * n * stride, -1)
        cache_v = mla.kv_cache(mla.BF16, rows.contiguous(), row_stride=d.width, seq_stride=stride)
    o_d, l_d = _decode_rows(pipe, cache_v, _visible(inp.seq_lens, n))
    assert torch.equal(o_m, o_d) and torch.equal(l_m, l_d)
    del cache_v, o_d
    out, lse = pipe.run()
    torch.cuda.synchronize()
    out, lse = out.double().cpu().numpy(), lse.double().cpu().numpy()
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    _sampled_oracle(inp, out, lse, [0, 1, 17, 40, 63], n)
