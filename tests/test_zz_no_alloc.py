"""mq_linear_noalloc (split-k workspace from the library's static per-device
scratch) against mq_linear with a caller workspace, through the C ABI: two
calls in a row, the second with a smaller input, each bit for bit equal to the
existing entry point and within tolerance of the fp64 oracle."""
import numpy as np
import pytest
import torch

from oracle import mq_oracle as O
from nested_integer_weight_amd import _lib, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def mq():
    from nested_integer_weight_amd import mq as _mq
    return _mq


def _case(mq, tid, m, n, k, group, dt):
    lay = synth.make_layer(cfg_id=11, tensor_id=tid, n=n, k=k, m=m, group=group, x_dtype=dt)
    q = torch.from_numpy(lay.q).to(DEV)
    s = torch.from_numpy(lay.scales).to(DEV)
    z = torch.from_numpy(lay.zeros).to(DEV)
    return lay, mq.pack_parent(q), s, z, lay.x.to(DEV)


def _check(mq, lay, pk, s, z, x, r, rule):
    m, n = x.shape[0], pk.n
    ws = mq.Workspace()
    assert mq.workspace_bytes(m, n, pk.k) > 0  # the shape splits k
    ref = mq.linear(x, pk, r, rule, lay.group, s, z, workspace=ws)
    out = torch.full((m, n), float("nan"), dtype=x.dtype, device=DEV)
    mq.linear_noalloc(x, pk, r, rule, lay.group, s, z, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    x64 = lay.x.double().numpy()
    w64 = O.dequant(lay.q, lay.scales, lay.zeros, r, rule, lay.group)
    err = O.normalized_error(out.float().cpu().numpy(), x64 @ w64.T, x64, w64)
    assert err <= 2e-3, err


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_noalloc_two_calls_second_smaller(mq, dt):
    # skinny path with a k split (7 MiB of partial sums), then a smaller one
    big = _case(mq, 1, 64, 4096, 14336, 128, dt)
    small = _case(mq, 2, 24, 512, 4096, 128, dt)
    _check(mq, *big, 3, O.PREFIX)
    _check(mq, *small, 3, O.PREFIX)


def test_noalloc_gemm_split_then_smaller(mq):
    # prefill GEMM with a k split, then a smaller GEMM and a skinny call
    a = _case(mq, 3, 300, 448, 1024, 128, "bf16")
    b = _case(mq, 4, 257, 320, 1024, 64, "f16")
    c = _case(mq, 5, 16, 320, 1024, 128, "f16")
    _check(mq, *a, 8, O.ROUND)
    _check(mq, *b, 4, O.PREFIX)
    _check(mq, *c, 2, O.PREFIX)
