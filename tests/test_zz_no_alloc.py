"""The allocation-free cache append (mla_cache_append_noalloc) against the
workspace form (mla_cache_append): the same kernels, the partial sums in the
library's own per-GPU scratch instead of the caller's workspace, so the rows
written are the same bits. Two calls in a row, the second with fewer
sequences (the scratch keeps the first call's contents), for a bf16 and an
e4m3 cache and the tiny fp32 shape; a call beyond the scratch is refused
before anything is enqueued."""

import numpy as np
import pytest
import torch

from mla_synth import DSV2, TINY, make_append_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_28_amd as mla
    mla.lib()     # fails loudly when the library is missing


def _cache(mla, d, B, cap, kind, dev="cuda"):
    width = d.d_latent + d.d_rope
    if kind == "fp8":
        codes = torch.full((B * cap, d.d_latent), 0x55, dtype=torch.uint8, device=dev)
        scale = torch.full((B * cap,), -1.0, dtype=torch.float32, device=dev)
        rope = torch.full((B * cap, d.d_rope), float("nan"), dtype=torch.bfloat16, device=dev)
        return (codes, scale, rope), mla.kv_cache(mla.FP8_E4M3, codes, rope=rope, scale=scale,
                                                  row_stride=d.d_latent, rope_stride=d.d_rope, seq_stride=cap)
    t = torch.float32 if kind == "f32" else torch.bfloat16
    rows = torch.full((B * cap, width), float("nan"), dtype=t, device=dev)
    return (rows,), mla.kv_cache(mla.F32 if kind == "f32" else mla.BF16, rows, row_stride=width, seq_stride=cap)


@pytest.mark.parametrize("kind", ["bf16", "fp8", "f32"])
def test_noalloc_append_equals_workspace_append(kind):
    import mla_latent_kv_28_amd as mla
    d = TINY if kind == "f32" else DSV2
    dt = mla.F32 if kind == "f32" else mla.BF16
    cap = 48
    for call, B in enumerate((64, 9)):            # the second call is smaller
        inp = make_append_inputs(d, batch=B, seed=20 + call, max_position=cap, with_gain=(call == 0))
        print("case: noalloc append kind=%s call=%d B=%d" % (kind, call, B), flush=True)
        args = lambda: (d, B, d.hidden, inp.h.cuda(), inp.w_dkv.cuda(), inp.w_kr.cuda(),
                        None if inp.gain is None else inp.gain.cuda(), dt, inp.eps, inp.base,
                        torch.from_numpy(inp.positions).cuda())
        ref_store, ref_cache = _cache(mla, d, B, cap, kind)
        ws = torch.empty(mla.mla_cache_append_workspace(d, B, d.hidden) // 4, dtype=torch.float32, device="cuda")
        mla.mla_cache_append(*args(), ref_cache, ws)
        got_store, got_cache = _cache(mla, d, B, cap, kind)
        mla.mla_cache_append_noalloc(*args(), got_cache)
        torch.cuda.synchronize()
        for r, g in zip(ref_store, got_store):          # bit for bit, NaN fill included
            assert torch.equal(r.view(torch.uint8), g.view(torch.uint8))
        assert np.all((inp.positions >= 0) & (inp.positions < cap))   # every sequence got its row


def test_noalloc_append_refuses_a_batch_beyond_the_scratch():
    import mla_latent_kv_28_amd as mla
    B = 800                                        # 800 x 5 parts x 576 x 4 bytes > 8 MiB
    assert mla.mla_cache_append_workspace(DSV2, B, DSV2.hidden) > (8 << 20)
    inp = make_append_inputs(DSV2, batch=B, seed=3, max_position=4)
    store, cache = _cache(mla, DSV2, B, 4, "bf16")
    with pytest.raises(mla.MLAError) as e:
        mla.mla_cache_append_noalloc(DSV2, B, DSV2.hidden, inp.h.cuda(), inp.w_dkv.cuda(), inp.w_kr.cuda(), None,
                                     mla.BF16, inp.eps, inp.base, torch.from_numpy(inp.positions).cuda(), cache)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert torch.isnan(store[0].float()).all()     # nothing was written
