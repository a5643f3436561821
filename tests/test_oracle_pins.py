"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes one part of the oracle by something independent of its code:
a brute-force evaluation of the definition on tiny inputs, a library routine
(torch's scaled_dot_product_attention, torch's float8 cast), closed forms and
special cases with a known answer, and the numbers the pages print.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from mla_synth import make_inputs, oracle_args

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _rand_case(rng, H=4, L=37, d_c=32, d_nope=24, d_r=16, d_v=20):
    """Random float64 case with every width distinct, so a transposed or
    swapped operand cannot pass silently on shape alone."""
    return dict(
        c_kv=rng.standard_normal((L, d_c)),
        k_rope=rng.standard_normal((L, d_r)),
        q_nope=rng.standard_normal((H, d_nope)),
        q_rope=rng.standard_normal((H, d_r)),
        w_uk=rng.standard_normal((H, d_nope, d_c)) / math.sqrt(d_c),
        w_uv=rng.standard_normal((H, d_v, d_c)) / math.sqrt(d_c),
        sm_scale=1.0 / math.sqrt(d_nope + d_r),
    )


def _rel(a, b):
    return float(np.linalg.norm(np.ravel(a - b)) / np.linalg.norm(np.ravel(b)))


# --- P1: absorbed and non-absorbed forms agree --------------------------------

def test_absorbed_equals_nonabsorbed_tiny_workload():
    inp = make_inputs("tiny")
    a = oracle_args(inp)
    c_kv, k_rope = oracle.gather_rows(a["cache"], 0, int(inp.seq_lens[0]))
    o1, l1 = oracle.attend_nonabsorbed(c_kv, k_rope, a["q_nope"][0], a["q_rope"][0],
                                       a["w_uk"], a["w_uv"], a["sm_scale"])
    o2, l2, _ = oracle.attend_absorbed(c_kv, k_rope, a["q_nope"][0], a["q_rope"][0],
                                       a["w_uk"], a["w_uv"], a["sm_scale"])
    assert _rel(o1, o2) <= 1e-5
    assert _rel(o1, o2) <= 1e-12          # holds far below the required 1e-5
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_absorbed_equals_nonabsorbed_dsv2_shapes():
    inp = make_inputs("dsv2_b32_l4096", batch=1, seq_lens=[77])
    a = oracle_args(inp)
    c_kv, k_rope = oracle.gather_rows(a["cache"], 0, 77)
    o1, l1 = oracle.attend_nonabsorbed(c_kv, k_rope, a["q_nope"][0], a["q_rope"][0],
                                       a["w_uk"], a["w_uv"], a["sm_scale"])
    o2, l2, _ = oracle.attend_absorbed(c_kv, k_rope, a["q_nope"][0], a["q_rope"][0],
                                       a["w_uk"], a["w_uv"], a["sm_scale"])
    assert _rel(o1, o2) <= 1e-12
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


# --- P2: brute force from the definition, pure Python ------------------------

def _brute_force(case):
    """Attention evaluated straight from the definition with Python floats:
    k_{j,h}[i] = sum_c W_UK[h][i][c] c_j[c], then [k; k^R]; v likewise with
    W_UV and no rotary part; p_j = exp(s_j) / sum exp(s_i) without any max
    subtraction; o = sum_j p_j v_j; lse = log sum exp(s_i)."""
    c_kv = case["c_kv"].tolist()
    k_rope = case["k_rope"].tolist()
    w_uk = case["w_uk"].tolist()
    w_uv = case["w_uv"].tolist()
    L = len(c_kv)
    out, lses = [], []
    for h in range(len(w_uk)):
        q = case["q_nope"][h].tolist() + case["q_rope"][h].tolist()
        scores, values = [], []
        for j in range(L):
            k = [math.fsum(w_uk[h][i][c] * c_kv[j][c] for c in range(len(c_kv[j])))
                 for i in range(len(w_uk[h]))] + k_rope[j]
            v = [math.fsum(w_uv[h][i][c] * c_kv[j][c] for c in range(len(c_kv[j])))
                 for i in range(len(w_uv[h]))]
            scores.append(case["sm_scale"] * math.fsum(a * b for a, b in zip(q, k)))
            values.append(v)
        e = [math.exp(s) for s in scores]
        z = math.fsum(e)
        out.append([math.fsum(e[j] / z * values[j][i] for j in range(L))
                    for i in range(len(values[0]))])
        lses.append(math.log(z))
    return np.array(out), np.array(lses)


def test_oracle_matches_brute_force_definition():
    case = _rand_case(np.random.default_rng(11))
    o_bf, l_bf = _brute_force(case)
    o, l = oracle.attend_nonabsorbed(**case)
    np.testing.assert_allclose(o, o_bf, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l, l_bf, rtol=1e-13, atol=0)
    # the softmax weights sum to one: recover them from a constant value row
    case1 = dict(case)
    case1["w_uv"] = np.zeros_like(case["w_uv"])
    assert np.all(oracle.attend_nonabsorbed(**case1)[0] == 0)


# --- P3: per-head attention equals a library routine ---------------------------

def test_oracle_matches_torch_sdpa():
    case = _rand_case(np.random.default_rng(5), H=3, L=53)
    o, lse = oracle.attend_nonabsorbed(**case)
    c = torch.from_numpy(case["c_kv"])
    for h in range(3):
        kc = c @ torch.from_numpy(case["w_uk"][h]).T              # [L, d_nope]
        k = torch.cat([kc, torch.from_numpy(case["k_rope"])], 1)  # [L, d_nope + d_r]
        v = c @ torch.from_numpy(case["w_uv"][h]).T               # [L, d_v]
        q = torch.cat([torch.from_numpy(case["q_nope"][h]), torch.from_numpy(case["q_rope"][h])])
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[None, None, None], k[None, None], v[None, None], scale=case["sm_scale"])
        np.testing.assert_allclose(o[h], ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[h], torch.logsumexp(case["sm_scale"] * (k @ q), 0).item(),
                                   rtol=1e-14, atol=0)


# --- P4: closed forms printed on the pages -------------------------------------

def test_closed_forms_match_printed_numbers():
    items = {it["name"]: it for it in json.load(open(GOLDEN))["items"]}
    it = items["mla_cache_elements_per_token_per_layer"]
    assert oracle.cache_elements_per_token(**it["inputs"]) == it["value"]
    it = items["mha_elements_per_token_per_layer"]
    assert oracle.mha_elements_per_token(**it["inputs"]) == it["value"]
    it = items["gqa_equivalent_groups"]
    d_h = it["inputs"]["d_h"]
    g = oracle.gqa_equivalent_groups(it["inputs"]["d_c_over_d_h"] * d_h,
                                     int(it["inputs"]["d_rope_over_d_h"] * d_h), d_h)
    assert g == it["value"]
    it = items["kv_cache_reduction_vs_deepseek_67b_percent"]
    x = it["inputs"]
    red = oracle.kv_reduction_vs_gqa_model(512, 64, x["mla_layers"], x["mla_bits"],
                                           x["gqa_groups"], x["d_h"], x["gqa_layers"],
                                           x["gqa_bits"])
    assert round(100 * red, it["rounding"]) == it["value"]
    # the same ratio without the cache quantisation is far from the printed value
    red16 = oracle.kv_reduction_vs_gqa_model(512, 64, 60, 16, 8, 128, 95, 16)
    assert abs(100 * red16 - 82.2) < 0.05


def test_bf16_row_bytes():
    # 576 bf16 elements per token: 1152 bytes; the fp8 layout keeps 512 one-byte
    # codes, a 64-wide bf16 rotary key and one fp32 scale: 644 bytes.
    assert oracle.cache_elements_per_token(512, 64) * 2 == 1152
    inp = make_inputs("fp8_b128_l8192", batch=1, seq_lens=[3])
    assert inp.cache_bytes() == 3 * 644


# --- P5-P7: special cases with a closed-form answer -----------------------------

def test_single_token_returns_projected_latent():
    case = _rand_case(np.random.default_rng(1), L=1)
    o, lse = oracle.attend_nonabsorbed(**case)
    for h in range(case["w_uv"].shape[0]):
        np.testing.assert_allclose(o[h], case["w_uv"][h] @ case["c_kv"][0], rtol=1e-13, atol=1e-15)
        s0 = case["sm_scale"] * (np.dot(case["w_uk"][h] @ case["c_kv"][0], case["q_nope"][h])
                                 + np.dot(case["k_rope"][0], case["q_rope"][h]))
        assert abs(lse[h] - s0) <= 1e-13 * max(1.0, abs(s0))


def test_zero_query_is_uniform_average():
    case = _rand_case(np.random.default_rng(2), L=29)
    case["q_nope"][:] = 0
    case["q_rope"][:] = 0
    o, lse = oracle.attend_nonabsorbed(**case)
    mean_c = case["c_kv"].mean(axis=0)
    for h in range(o.shape[0]):
        np.testing.assert_allclose(o[h], case["w_uv"][h] @ mean_c, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(29), rtol=1e-14)


def test_identical_rows_give_that_row():
    case = _rand_case(np.random.default_rng(3), L=17)
    case["c_kv"][:] = case["c_kv"][4]
    case["k_rope"][:] = case["k_rope"][4]
    o, lse = oracle.attend_nonabsorbed(**case)
    for h in range(o.shape[0]):
        np.testing.assert_allclose(o[h], case["w_uv"][h] @ case["c_kv"][0], rtol=1e-12, atol=1e-14)


def test_very_large_scale_selects_argmax_row():
    case = _rand_case(np.random.default_rng(4), L=23)
    case["sm_scale"] = 1e4
    o, _ = oracle.attend_nonabsorbed(**case)
    for h in range(o.shape[0]):
        s = (case["c_kv"] @ (case["w_uk"][h].T @ case["q_nope"][h])
             + case["k_rope"] @ case["q_rope"][h])
        j = int(np.argmax(s))
        np.testing.assert_allclose(o[h], case["w_uv"][h] @ case["c_kv"][j], rtol=1e-9, atol=1e-12)


def test_empty_cache():
    case = _rand_case(np.random.default_rng(4), L=0)
    o, lse = oracle.attend_nonabsorbed(**case)
    assert np.all(o == 0) and np.all(lse == -np.inf)


# --- P8: token order does not matter (pins the paged gather) ----------------------

def test_permutation_invariance():
    case = _rand_case(np.random.default_rng(6), L=41)
    o, lse = oracle.attend_nonabsorbed(**case)
    perm = np.random.default_rng(7).permutation(41)
    case["c_kv"] = case["c_kv"][perm]
    case["k_rope"] = case["k_rope"][perm]
    o2, lse2 = oracle.attend_nonabsorbed(**case)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-14)


def test_paged_and_contiguous_layouts_agree():
    lens = [130, 64, 1, 77]
    a = oracle_args(make_inputs("dsv2_b32_l4096", batch=4, seq_lens=lens, pad_fill=float("nan")))
    p = oracle_args(make_inputs("dsv2_b32_l4096", batch=4, seq_lens=lens, layout="paged",
                                page_size=64, pad_fill=float("nan")))
    assert p["cache"]["block_table"].shape == (4, 3)
    o1, l1 = oracle.decode(**a)
    o2, l2 = oracle.decode(**p)
    assert np.all(np.isfinite(o1))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def _glue_case(rng, lens, H=3, d_c=12, d_nope=8, d_r=6, d_v=10):
    """A small batch whose every sequence has its own rows and its own query,
    so that an indexing slip (a sequence reading another's rows, or another's
    query) changes the result."""
    B = len(lens)
    return dict(
        q_nope=rng.standard_normal((B, H, d_nope)),
        q_rope=rng.standard_normal((B, H, d_r)),
        w_uk=rng.standard_normal((H, d_nope, d_c)) / math.sqrt(d_c),
        w_uv=rng.standard_normal((H, d_v, d_c)) / math.sqrt(d_c),
        sm_scale=1.0 / math.sqrt(d_nope + d_r),
    ), d_c, d_r


def test_batched_decode_equals_attention_on_hand_sliced_rows():
    # oracle.decode is glue: gather each sequence's rows, attend with that
    # sequence's query. Rows are placed by hand here (contiguous: sequence b at
    # rows b * stride ..; paged: pages taken from a hand-written table) and the
    # attention of each sequence is taken on exactly those rows.
    rng = np.random.default_rng(31)
    lens = [5, 0, 9, 1]
    args, d_c, d_r = _glue_case(rng, lens)
    stride = 11
    rows = np.full((len(lens) * stride, d_c + d_r), np.nan)
    per_seq = []
    for b, L in enumerate(lens):
        r = rng.standard_normal((L, d_c + d_r))
        rows[b * stride: b * stride + L] = r
        per_seq.append(r)
    page = 4
    table = np.array([[6, 1, 9], [0, 0, 0], [3, 8, 5], [2, 0, 0]], dtype=np.int32)
    pool = np.full((10 * page, d_c + d_r), np.nan)
    for b, L in enumerate(lens):
        for j in range(L):
            pool[table[b, j // page] * page + j % page] = per_seq[b][j]
    caches = [dict(kind="dense", d_c=d_c, rows=rows, seq_stride=stride),
              dict(kind="dense", d_c=d_c, rows=pool, block_table=table, page_size=page)]
    for cache in caches:
        o, lse = oracle.decode(cache=cache, seq_lens=np.array(lens), **args)
        for b, L in enumerate(lens):
            r = per_seq[b]
            ref_o, ref_l = oracle.attend_nonabsorbed(r[:, :d_c], r[:, d_c:], args["q_nope"][b],
                                                     args["q_rope"][b], args["w_uk"], args["w_uv"],
                                                     args["sm_scale"])
            np.testing.assert_array_equal(o[b], ref_o)
            np.testing.assert_array_equal(lse[b], ref_l)
        assert np.all(o[1] == 0) and np.all(lse[1] == -np.inf)
        # every sequence's result differs from the others' (distinct queries and rows)
        for b in (0, 2, 3):
            for c in (0, 2, 3):
                if b != c:
                    assert not np.allclose(o[b], o[c])


def test_decode_one_and_heads_equal_batched_decode():
    # the single-(sequence, head) and head-subset forms used for the checks at
    # full size give the same values as the batched call, head by head
    rng = np.random.default_rng(32)
    lens = [7, 3, 12]
    args, d_c, d_r = _glue_case(rng, lens, H=4)
    stride = 12
    rows = rng.standard_normal((len(lens) * stride, d_c + d_r))
    cache = dict(kind="dense", d_c=d_c, rows=rows, seq_stride=stride)
    o, lse = oracle.decode(cache=cache, seq_lens=np.array(lens), **args)
    for b in range(len(lens)):
        for h in range(4):
            o1, l1 = oracle.decode_one(cache=cache, seq_lens=np.array(lens), b=b, h=h, **args)
            np.testing.assert_allclose(o1, o[b, h], rtol=1e-13, atol=1e-15)
            assert abs(l1 - lse[b, h]) <= 1e-13 * max(1.0, abs(lse[b, h]))
        hs = [3, 0, 2]
        oh, lh = oracle.decode_heads(cache=cache, seq_lens=np.array(lens), b=b, heads=hs, **args)
        np.testing.assert_allclose(oh, o[b, hs], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(lh, lse[b, hs], rtol=1e-13, atol=0)


def test_fp8_cache_gather_equals_dense_cache_of_library_decoded_codes():
    # the e4m3 branch of the gather (codes decoded by the oracle's own table,
    # times the per-token scale) against a dense cache whose latent values come
    # from torch's float8_e4m3fn -> float32 conversion, times the scale in float64
    rng = np.random.default_rng(33)
    lens = [6, 9]
    args, d_c, d_r = _glue_case(rng, lens)
    R = 20
    codes = rng.integers(0, 256, size=(R, d_c)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C          # no NaN codes
    scale = (rng.random(R) * 0.02 + 1e-3).astype(np.float32)
    rope = rng.standard_normal((R, d_r)).astype(np.float32)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    dense_rows = np.concatenate([lib * scale.astype(np.float64)[:, None], rope], axis=1)
    fp8 = dict(kind="fp8", d_c=d_c, codes=codes, scale=scale, rope=rope, seq_stride=10)
    dense = dict(kind="dense", d_c=d_c, rows=dense_rows, seq_stride=10)
    for b, L in enumerate(lens):
        c8, r8 = oracle.gather_rows(fp8, b, L)
        cd, rd = oracle.gather_rows(dense, b, L)
        np.testing.assert_array_equal(c8, cd)
        np.testing.assert_array_equal(r8, rd)
    o8, l8 = oracle.decode(cache=fp8, seq_lens=np.array(lens), **args)
    od, ld = oracle.decode(cache=dense, seq_lens=np.array(lens), **args)
    np.testing.assert_array_equal(o8, od)
    np.testing.assert_array_equal(l8, ld)


def test_token_rows_paged_mapping():
    bt = np.array([[5, 2, 7], [0, 1, 3]], dtype=np.int32)
    rows = oracle.mla.token_rows(0, 10, block_table=bt, page_size=4)
    assert rows.tolist() == [20, 21, 22, 23, 8, 9, 10, 11, 28, 29]
    rows = oracle.mla.token_rows(1, 3, seq_stride=100)
    assert rows.tolist() == [100, 101, 102]


# --- P9: split-KV with log-sum-exp merge equals the unsplit result ---------------

@pytest.mark.parametrize("bounds", [[0, 60], [0, 1, 60], [0, 13, 13, 40, 60], [0, 30, 60, 60]])
def test_split_merge_invariance(bounds):
    case = _rand_case(np.random.default_rng(8), L=60)
    o, lse = oracle.attend_nonabsorbed(**case)
    o2, lse2 = oracle.attend_split(bounds=bounds, **case)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)


def test_merge_of_only_empty_parts():
    o, lse = oracle.lse_merge(np.zeros((3, 2, 5)), np.full((3, 2), -np.inf))
    assert np.all(o == 0) and np.all(lse == -np.inf)


# --- P10: e4m3 codec ----------------------------------------------------------

def test_e4m3_table_against_definition_values():
    t = oracle.e4m3_table()
    assert t[0x7E] == 448.0                # largest finite
    assert t[0x08] == 2.0 ** -6            # smallest normal
    assert t[0x01] == 2.0 ** -9            # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert t[0x38] == 1.0
    assert t[0x3C] == 1.5
    assert t[0xB8] == -1.0
    assert t[0x80] == 0.0 and math.copysign(1.0, t[0x80]) == -1.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    got = oracle.decode_e4m3(np.arange(256))
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_e4m3_encode_matches_torch_cast():
    t = oracle.e4m3_table()
    finite = t[np.isfinite(t)]
    mids = (np.sort(finite)[1:] + np.sort(finite)[:-1]) / 2      # exact ties
    x = np.concatenate([np.linspace(-448, 448, 100001), finite, mids,
                        mids * (1 + 1e-6), mids * (1 - 1e-6), [0.0, -0.0, 1e-30, -1e-30]])
    # torch rounds a float64 source to float32 before the fp8 cast, so compare
    # on float32 inputs, which is what the cache quantiser feeds it.
    x = x.astype(np.float32)
    got = oracle.encode_e4m3(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, ref)
    # saturation beyond the range (torch's cast does not saturate; clamp first)
    assert oracle.encode_e4m3(np.array([1e6, -500.0])).tolist() == [0x7E, 0xFE]


def test_e4m3_quantised_cache_matches_codec():
    inp = make_inputs("fp8_b128_l8192", batch=1, seq_lens=[40])
    codes = inp.codes.numpy()
    scale = inp.scale.numpy().astype(np.float64)
    c = inp.rows[:40, :512].double().numpy()
    # the quantiser divides in float32
    y = (inp.rows[:40, :512].float() / inp.scale[:40, None]).double().numpy()
    np.testing.assert_array_equal(oracle.encode_e4m3(y), codes[:40])
    assert np.all((codes[:40] & 0x7F).max(axis=1) == 0x7E)   # the absmax element -> 448
    deq = oracle.decode_e4m3(codes[:40]) * scale[:40, None]
    # e4m3 keeps 3 mantissa bits: relative error at most 2^-4 for normals
    big = np.abs(c) > 2.0 ** -6 * scale[:40, None]
    assert np.all(np.abs(deq - c)[big] <= 2.0 ** -4 * np.abs(c)[big])


# --- softmax scales of the workloads ---------------------------------------------

def test_workload_softmax_scales():
    assert make_inputs("tiny").sm_scale == pytest.approx(1 / math.sqrt(48), rel=1e-15)
    assert make_inputs("dsv2_b32_l4096", batch=1, seq_lens=[2]).sm_scale == \
        pytest.approx(1 / math.sqrt(192), rel=1e-15)
    long = make_inputs("long_b4_l131072", batch=1, seq_lens=[2]).sm_scale
    assert long == pytest.approx(0.0987910, abs=5e-8)


# --- the cache entry of a new token (latent, rotary key, e4m3 form) --------------

def test_rms_norm_closed_forms_and_library():
    # a constant row normalises to +-1 (eps 0); [3, 4] has mean square 12.5
    assert np.allclose(oracle.rms_norm(np.full(7, -2.5), 0.0), -1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(oracle.rms_norm(np.array([3.0, 4.0]), 0.0),
                               np.array([3.0, 4.0]) / math.sqrt(12.5), rtol=1e-15)
    rng = np.random.default_rng(3)
    x, g = rng.standard_normal((5, 96)), rng.standard_normal(96)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), 1e-6).numpy()
    np.testing.assert_allclose(oracle.rms_norm(x, 1e-6, g), ref, rtol=1e-13, atol=1e-13)


def test_rope_closed_forms_and_relative_position():
    # one pair at frequency 1: position 1 turns (1, 0) by one radian
    np.testing.assert_allclose(oracle.rope(np.array([1.0, 0.0]), 1, 10000.0),
                               [math.cos(1.0), math.sin(1.0)], rtol=0, atol=1e-15)
    # d = 4, base 10000: the second pair turns at 10000^(-1/2) = 0.01 rad per position
    np.testing.assert_allclose(oracle.rope(np.array([0.0, 0.0, 0.0, 1.0]), 100, 10000.0),
                               [0.0, 0.0, -math.sin(1.0), math.cos(1.0)], rtol=0, atol=1e-14)
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    assert np.array_equal(oracle.rope(q, 0, 10000.0), q)                      # position 0: identity
    for m in (0, 7, 4095):
        assert np.linalg.norm(oracle.rope(q, m, 10000.0)) == pytest.approx(np.linalg.norm(q), rel=1e-14)
    # the defining property: the score of rotated q and k depends on m - n only
    s1 = oracle.rope(q, 1000, 10000.0) @ oracle.rope(k, 990, 10000.0)
    s2 = oracle.rope(q, 20, 10000.0) @ oracle.rope(k, 10, 10000.0)
    assert s1 == pytest.approx(s2, rel=1e-11)
    s3 = oracle.rope(q, 21, 10000.0) @ oracle.rope(k, 10, 10000.0)
    assert abs(s3 - s2) > 1e-3                                                  # and does depend on it


def test_append_entry_brute_force_and_one_hot():
    rng = np.random.default_rng(5)
    B, d, d_c, d_r = 3, 12, 8, 4
    h = rng.standard_normal((B, d))
    w_dkv, w_kr = rng.standard_normal((d_c, d)), rng.standard_normal((d_r, d))
    gain, pos, eps, base = rng.standard_normal(d_c), np.array([0, 5, 130]), 1e-6, 500.0
    c, k = oracle.append_entry(h, w_dkv, w_kr, pos, eps, base, gain)
    for b in range(B):                      # the definition in plain loops
        x = [sum(w_dkv[i, j] * h[b, j] for j in range(d)) for i in range(d_c)]
        ms = sum(v * v for v in x) / d_c
        for i in range(d_c):
            assert c[b, i] == pytest.approx(x[i] / math.sqrt(ms + eps) * gain[i], rel=1e-12)
        y = [sum(w_kr[i, j] * h[b, j] for j in range(d)) for i in range(d_r)]
        for i in range(d_r // 2):
            a = pos[b] * base ** (-2.0 * i / d_r)
            assert k[b, 2 * i] == pytest.approx(y[2 * i] * math.cos(a) - y[2 * i + 1] * math.sin(a), rel=1e-11, abs=1e-12)
            assert k[b, 2 * i + 1] == pytest.approx(y[2 * i] * math.sin(a) + y[2 * i + 1] * math.cos(a), rel=1e-11, abs=1e-12)
    # a one-hot hidden state selects a column of each projection
    e = np.zeros((1, d))
    e[0, 4] = 2.0
    c1, k1 = oracle.append_entry(e, w_dkv, w_kr, [0], 0.0, base)
    col = 2.0 * w_dkv[:, 4]
    np.testing.assert_allclose(c1[0], col / np.sqrt(np.mean(col ** 2)), rtol=1e-14)
    np.testing.assert_allclose(k1[0], 2.0 * w_kr[:, 4], rtol=1e-14)


def test_quantise_entry_against_library_cast():
    rng = np.random.default_rng(6)
    c = rng.standard_normal((4, 512)) * np.array([1.0, 1e-3, 30.0, 0.0])[:, None]
    codes, scale = oracle.quantise_entry(c)
    assert scale[3] == 1.0 and np.all(codes[3] & 0x7F == 0)                  # all-zero row (signed zeros)
    np.testing.assert_allclose(scale[:3], np.abs(c[:3]).max(axis=1) / 448.0, rtol=1e-15)
    y = np.clip(c[:3] / scale[:3, None], -448.0, 448.0)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes[:3], ref)
    assert np.all((codes[:3] & 0x7F).max(axis=1) == 0x7E)                     # the absmax element is 448


# --- the attention output projection -----------------------------------------------

def test_output_projection_brute_force_one_hot_and_absorption():
    rng = np.random.default_rng(8)
    B, H, d_v, d_c, hid = 2, 3, 4, 5, 6
    o, w_o = rng.standard_normal((B, H, d_v)), rng.standard_normal((hid, H * d_v))
    u = oracle.output_projection(o, w_o)
    for b in range(B):                              # the definition in plain loops
        for i in range(hid):
            ref = sum(w_o[i, h * d_v + j] * o[b, h, j] for h in range(H) for j in range(d_v))
            assert u[b, i] == pytest.approx(ref, rel=1e-13, abs=1e-13)
    e = np.zeros((1, H, d_v))                       # one head's feature selects one column
    e[0, 2, 1] = 1.0
    np.testing.assert_array_equal(oracle.output_projection(e, w_o)[0], w_o[:, 2 * d_v + 1])
    # W_UV folded into W_O (V2 2.1.2) gives the same output from the latent outputs
    w_uv, o_lat = rng.standard_normal((H, d_v, d_c)), rng.standard_normal((B, H, d_c))
    o2 = np.einsum("hvc,bhc->bhv", w_uv, o_lat)
    folded = np.concatenate([w_o[:, h * d_v:(h + 1) * d_v] @ w_uv[h] for h in range(H)], axis=1)
    np.testing.assert_allclose(oracle.output_projection(o2, w_o), o_lat.reshape(B, -1) @ folded.T,
                               rtol=1e-12, atol=1e-12)


# --- the query path and the rotary frequencies (plain and YaRN) -----------------------

def _pair_angles(freqs_rotation, d):
    """Angle by which each pair of a unit vector turns at position 1, read off
    the rotated vector (atan2), so frequencies are compared through rotations."""
    out = []
    for i in range(d // 2):
        e = np.zeros(d)
        e[2 * i] = 1.0
        r = freqs_rotation(e)
        out.append(math.atan2(r[2 * i + 1], r[2 * i]))
    return np.array(out)


def test_rope_frequencies_plain_equal_rope_and_yarn_limits():
    rng = np.random.default_rng(41)
    d, base = 64, 10000.0
    x = rng.standard_normal((3, d))
    pos = np.array([0, 17, 4095])
    plain = oracle.rope_frequencies(d, base)
    np.testing.assert_allclose(oracle.rope_with(x, pos, plain), oracle.rope(x, pos, base), rtol=0, atol=1e-12)
    # every pair "long" against the original context: each frequency divided by
    # s, i.e. position interpolation: turning at p with theta / s = turning at p / s
    s = 40.0
    interp = oracle.rope_frequencies(d, base, s, yarn_alpha=1e12, yarn_beta=2e12)
    np.testing.assert_allclose(oracle.rope_with(x, pos, interp), oracle.rope(x, pos / s, base), rtol=0, atol=1e-12)
    # every pair "short": no change
    keep = oracle.rope_frequencies(d, base, s, yarn_alpha=-2.0, yarn_beta=-1.0)
    np.testing.assert_allclose(keep, plain, rtol=0, atol=0)


def test_yarn_frequencies_with_the_pages_parameters():
    # s = 40, alpha = 1, beta = 32, original context 4096 (4K -> 160K), d_R = 64, base 10000
    d, base = 64, 10000.0
    f = oracle.rope_frequencies(d, base, 40.0, 1.0, 32.0, 4096)
    plain = _pair_angles(lambda e: oracle.rope(e, 1, base), d)       # plain angle per position, from rotations
    # turns of pair i over 4096 positions: pairs 0..10 turn more than 32 times
    # (their wavelengths 2 pi / theta_i are under 128 positions), 23..31 less than once
    turns = 4096 * plain / (2 * math.pi)
    assert np.all(turns[:11] > 32) and np.all(turns[23:] < 1) and np.all((turns[11:23] >= 1) & (turns[11:23] <= 32))
    np.testing.assert_allclose(f[:11], plain[:11], rtol=1e-13)          # high frequencies kept
    np.testing.assert_allclose(f[23:], plain[23:] / 40.0, rtol=1e-12)  # low ones interpolated by s
    assert np.all((f[11:23] < plain[11:23]) & (f[11:23] > plain[11:23] / 40.0))   # blended in between
    assert np.all(np.diff(f) < 0)                                       # still ordered
    # rotations with these frequencies keep the relative-position property
    rng = np.random.default_rng(42)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    s1 = oracle.rope_with(q, 100000, f) @ oracle.rope_with(k, 99000, f)
    s2 = oracle.rope_with(q, 1500, f) @ oracle.rope_with(k, 500, f)
    assert s1 == pytest.approx(s2, rel=1e-9)


def test_query_path_brute_force_one_hot_and_position_zero():
    rng = np.random.default_rng(43)
    B, d, dq, H, dn, dr = 2, 10, 6, 2, 3, 4
    h = rng.standard_normal((B, d))
    w_dq, w_uq, w_qr = rng.standard_normal((dq, d)), rng.standard_normal((H * dn, dq)), rng.standard_normal((H * dr, dq))
    gain, pos, eps = rng.standard_normal(dq), np.array([3, 250]), 1e-6
    f = oracle.rope_frequencies(dr, 500.0, 8.0, 1.0, 4.0, orig_ctx=64)
    c, qn, qr = oracle.query_path(h, w_dq, w_uq, w_qr, pos, eps, f, H, gain)
    angles = _pair_angles(lambda e: oracle.rope_with(e, 1, f), dr)
    for b in range(B):                       # the definition in plain loops
        x = [sum(w_dq[i, j] * h[b, j] for j in range(d)) for i in range(dq)]
        rms = math.sqrt(sum(v * v for v in x) / dq + eps)
        cq = [x[i] / rms * gain[i] for i in range(dq)]
        for i in range(dq):
            assert c[b, i] == pytest.approx(cq[i], rel=1e-12)
        for hh in range(H):
            for n in range(dn):
                assert qn[b, hh, n] == pytest.approx(sum(w_uq[hh * dn + n, i] * cq[i] for i in range(dq)), rel=1e-11, abs=1e-12)
            y = [sum(w_qr[hh * dr + n, i] * cq[i] for i in range(dq)) for n in range(dr)]
            for i in range(dr // 2):
                a = pos[b] * angles[i]
                assert qr[b, hh, 2 * i] == pytest.approx(y[2 * i] * math.cos(a) - y[2 * i + 1] * math.sin(a), rel=1e-10, abs=1e-11)
                assert qr[b, hh, 2 * i + 1] == pytest.approx(y[2 * i] * math.sin(a) + y[2 * i + 1] * math.cos(a), rel=1e-10, abs=1e-11)
    # a one-hot hidden state at position 0: c_Q is the normed column, the
    # queries the up-projections of it, unrotated
    e = np.zeros((1, d))
    e[0, 7] = -3.0
    c1, qn1, qr1 = oracle.query_path(e, w_dq, w_uq, w_qr, [0], 0.0, f, H)
    col = -3.0 * w_dq[:, 7]
    np.testing.assert_allclose(c1[0], col / np.sqrt(np.mean(col ** 2)), rtol=1e-14)
    np.testing.assert_allclose(qn1[0].ravel(), w_uq @ c1[0], rtol=1e-13)
    np.testing.assert_allclose(qr1[0].ravel(), w_qr @ c1[0], rtol=1e-13)


def test_append_entry_with_frequencies():
    # the cache entry with explicit frequencies: plain ones reproduce the base
    # form; YaRN ones rotate the key as the query path rotates its queries
    rng = np.random.default_rng(44)
    h, w_dkv, w_kr = rng.standard_normal((3, 16)), rng.standard_normal((8, 16)), rng.standard_normal((4, 16))
    pos = np.array([0, 9, 300])
    c0, k0 = oracle.append_entry(h, w_dkv, w_kr, pos, 1e-6, 10000.0)
    c1, k1 = oracle.append_entry(h, w_dkv, w_kr, pos, 1e-6, 10000.0, freqs=oracle.rope_frequencies(4, 10000.0))
    np.testing.assert_array_equal(c0, c1)
    np.testing.assert_allclose(k1, k0, rtol=0, atol=1e-13)
    f = oracle.rope_frequencies(4, 10000.0, 40.0, 1.0, 32.0, 64)
    _, k2 = oracle.append_entry(h, w_dkv, w_kr, pos, 1e-6, 10000.0, freqs=f)
    np.testing.assert_allclose(k2, oracle.rope_with(h @ w_kr.T, pos, f), rtol=1e-13)
    np.testing.assert_allclose(k2[0], (h @ w_kr.T)[0], rtol=1e-15)     # position 0: unrotated


# --- several new tokens per sequence (causal over the appended tokens) ----------

def _multi_case(rng, lens, n, H=3, d_c=12, d_nope=8, d_r=6, d_v=10, stride=13):
    """Contiguous cache with sequence b at rows b * stride .., n queries per
    sequence (row b n + t), distinct widths."""
    B = len(lens)
    rows = np.full((B * stride, d_c + d_r), np.nan)
    for b, L in enumerate(lens):
        rows[b * stride:b * stride + L] = rng.standard_normal((L, d_c + d_r))
    cache = dict(kind="dense", rows=rows, d_c=d_c, seq_stride=stride)
    args = dict(
        q_nope=rng.standard_normal((B * n, H, d_nope)),
        q_rope=rng.standard_normal((B * n, H, d_r)),
        w_uk=rng.standard_normal((H, d_nope, d_c)) / math.sqrt(d_c),
        w_uv=rng.standard_normal((H, d_v, d_c)) / math.sqrt(d_c),
        cache=cache, seq_lens=np.array(lens, dtype=np.int32),
        sm_scale=1.0 / math.sqrt(d_nope + d_r),
    )
    return args, rows, d_c


def test_multi_token_zero_query_averages_its_causal_prefix():
    # q = 0: every visible row weighs the same, so token t of sequence b returns
    # W_UV times the mean latent of rows 0 .. L_b - n + t and lse = log(count);
    # a token that sees no row returns 0 and -inf
    n, lens = 3, [7, 1, 3, 12]
    args, rows, d_c = _multi_case(np.random.default_rng(41), lens, n)
    args["q_nope"][:] = 0
    args["q_rope"][:] = 0
    o, lse = oracle.decode_multi(n=n, **args)
    stride = args["cache"]["seq_stride"]
    for b, L in enumerate(lens):
        for t in range(n):
            count = L - n + t + 1
            bv = b * n + t
            if count <= 0:
                assert np.all(o[bv] == 0) and np.all(lse[bv] == -np.inf)
                continue
            mean_c = rows[b * stride:b * stride + count, :d_c].mean(axis=0)
            for h in range(o.shape[1]):
                np.testing.assert_allclose(o[bv, h], args["w_uv"][h] @ mean_c, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(lse[bv], math.log(count), rtol=1e-14)


def test_multi_token_mask_hides_later_tokens_only():
    # changing the row of token t + 1 (position L - n + t + 1) leaves tokens
    # 0 .. t of that sequence and every other sequence unchanged, and changes
    # tokens t + 1 .. n - 1
    n, lens = 4, [9, 6]
    args, rows, d_c = _multi_case(np.random.default_rng(42), lens, n)
    o0, l0 = oracle.decode_multi(n=n, **args)
    b, t = 1, 1
    pos = lens[b] - n + t + 1
    rows[b * args["cache"]["seq_stride"] + pos] += 3.0
    o1, l1 = oracle.decode_multi(n=n, **args)
    for bv in range(len(lens) * n):
        same = bv // n != b or bv % n <= t
        assert np.array_equal(o0[bv], o1[bv]) == same
        assert np.array_equal(l0[bv], l1[bv]) == same


def test_multi_token_last_token_and_single_token_equal_decode():
    # the last of the n tokens sees the whole sequence: it is `decode` with its
    # own query; n = 1 is `decode` itself
    n, lens = 3, [5, 11, 2]
    args, _, _ = _multi_case(np.random.default_rng(43), lens, n)
    o, lse = oracle.decode_multi(n=n, **args)
    last = dict(args, q_nope=args["q_nope"][n - 1::n], q_rope=args["q_rope"][n - 1::n])
    o_d, l_d = oracle.decode(**last)
    np.testing.assert_array_equal(o[n - 1::n], o_d)
    np.testing.assert_array_equal(lse[n - 1::n], l_d)
    args1, _, _ = _multi_case(np.random.default_rng(44), lens, 1)
    o1, l1 = oracle.decode_multi(n=1, **args1)
    o_d, l_d = oracle.decode(**args1)
    np.testing.assert_array_equal(o1, o_d)
    np.testing.assert_array_equal(l1, l_d)


def test_prefill_equals_multi_token_decode_and_brute_force():
    # prefill up-projects each sequence once and masks a score matrix; it must
    # reach the values of decode_multi (pinned above), also when a prefix of
    # older tokens precedes the n new ones and when a sequence is shorter than n
    n, lens = 5, [9, 5, 3, 14]
    args, rows, d_c = _multi_case(np.random.default_rng(45), lens, n, stride=16)
    o, lse = oracle.prefill(n=n, **args)
    o_m, l_m = oracle.decode_multi(n=n, **args)
    np.testing.assert_allclose(o, o_m, rtol=1e-12, atol=1e-14)
    assert np.array_equal(np.isfinite(lse), np.isfinite(l_m))
    np.testing.assert_allclose(lse[np.isfinite(lse)], l_m[np.isfinite(l_m)], rtol=1e-13)
    # brute force, one (row, head): pure-Python sums over the visible rows
    stride = args["cache"]["seq_stride"]
    b, t, h = 3, 2, 1
    L = lens[b]
    count = L - n + t + 1
    c = rows[b * stride:b * stride + count, :d_c]
    kr = rows[b * stride:b * stride + count, d_c:]
    qn, qr = args["q_nope"][b * n + t, h], args["q_rope"][b * n + t, h]
    sc = [args["sm_scale"] * (sum(qn[i] * sum(args["w_uk"][h][i][k] * c[j][k] for k in range(d_c))
                                   for i in range(len(qn))) + sum(qr[i] * kr[j][i] for i in range(len(qr))))
          for j in range(count)]
    w = [math.exp(x) for x in sc]
    z = sum(w)
    ref = [sum(w[j] / z * sum(args["w_uv"][h][v][k] * c[j][k] for k in range(d_c)) for j in range(count))
           for v in range(args["w_uv"].shape[1])]
    np.testing.assert_allclose(o[b * n + t, h], ref, rtol=1e-11, atol=1e-13)
    assert lse[b * n + t, h] == pytest.approx(math.log(z), rel=1e-12)
