"""GPU parity of the attention output projection (mla_o_proj) against the
float64 oracle. Bounds: fp32 output within 1e-5 relative L2 (bf16 inputs are
exact in fp32; only the fp32 sums round); bf16 output within 1e-2 relative L2
and 2^-8 relative plus 1e-4 absolute per element (one bf16 rounding); the
tiny fp32 shape within 1e-5.
"""

import numpy as np
import pytest
import torch

import oracle
from mla_synth import DSV2, TINY, make_oproj_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_28_amd as mla
    mla.lib()     # fails loudly when the library is missing


def _run(dims, batch, out_dtype, seed):
    import mla_latent_kv_28_amd as mla
    print("case: o_proj %s B=%d out=%s" % ("tiny" if dims == TINY else "dsv2", batch, out_dtype), flush=True)
    o, w_o = make_oproj_inputs(dims, batch, seed)
    dt = mla.F32 if dims == TINY else mla.BF16
    t = torch.float32 if out_dtype == mla.F32 else torch.bfloat16
    out = torch.full((batch, dims.hidden), float("nan"), dtype=t, device="cuda")
    nws = mla.mla_o_proj_workspace(dims, batch, dims.hidden)
    ws = torch.empty(max(nws // 4, 1), dtype=torch.float32, device="cuda") if nws else None
    mla.mla_o_proj(dims, batch, dims.hidden, o.cuda(), w_o.cuda(), dt, out, out_dtype, ws)
    torch.cuda.synchronize()
    ref = oracle.output_projection(o.double().numpy(), w_o.double().numpy())
    return out.double().cpu().numpy(), ref


def _rel(x, y):
    return float(np.linalg.norm((x - y).ravel()) / np.linalg.norm(y.ravel()))


@pytest.mark.parametrize("batch", [1, 32, 45])
def test_dsv2_f32_out(batch):
    import mla_latent_kv_28_amd as mla
    got, ref = _run(DSV2, batch, mla.F32, seed=batch)
    assert np.all(np.isfinite(got)) and _rel(got, ref) <= 1e-5


def test_dsv2_bf16_out():
    import mla_latent_kv_28_amd as mla
    got, ref = _run(DSV2, 32, mla.BF16, seed=3)
    assert _rel(got, ref) <= 1e-2
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4)


@pytest.mark.parametrize("hidden", [4096, 2048 + 128, 1024 + 32])
def test_dsv2_other_widths(hidden):
    # the 8-, 4- and 1-wave workgroups (160 does not divide these widths)
    import dataclasses
    import mla_latent_kv_28_amd as mla
    d = dataclasses.replace(DSV2, hidden=hidden)
    got, ref = _run(d, 7, mla.F32, seed=hidden)
    assert _rel(got, ref) <= 1e-5


def test_tiny_f32():
    import mla_latent_kv_28_amd as mla
    got, ref = _run(TINY, 3, mla.F32, seed=4)
    assert _rel(got, ref) <= 1e-5
