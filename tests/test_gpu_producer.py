"""The HIP parent producer (mq_produce_parent) against the CPU oracle.

Scales, zero points and codes are decisions taken in fp32 with the same
operations in the same order on both sides, so they must match bit for bit:
at small shapes that span several search blocks and a ragged last block, at
every rule and several width sets, candidate grids and lambda weightings, on
degenerate groups (all zero, constant, tiny, all negative, outliers), and on
sampled rows of a full Llama-3.1-8B FFN matrix.  The produced parent then runs
through packing and the layer and must give the oracle's Y."""
import numpy as np
import pytest
import torch

from oracle import mq_oracle as O
from oracle import mq_parent_oracle as P
from nested_integer_weight_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def mq():
    from nested_integer_weight_amd import mq as _mq
    return _mq


def produce_both(mq, w, group, widths, lams, rule, n_grid=80, grid_den=100):
    print(f"[producer] n={w.shape[0]} k={w.shape[1]} group={group} widths={widths} lambdas={lams} "
          f"rule={rule} grid={n_grid}/{grid_den}", flush=True)
    q, s, z = mq.produce_parent(torch.from_numpy(w).to(DEV), group, widths, lams, rule, n_grid, grid_den)
    torch.cuda.synchronize()
    q_ref, s_ref, z_ref = P.produce_parent(w, group, widths, lams, rule, n_grid, grid_den)
    return (q.cpu().numpy(), s.cpu().numpy(), z.cpu().numpy()), (q_ref, s_ref, z_ref)


def assert_same(got, ref):
    q, s, z = got
    q_ref, s_ref, z_ref = ref
    assert np.array_equal(s.view(np.uint16), s_ref.view(np.uint16)), \
        f"scales differ in {np.sum(s.view(np.uint16) != s_ref.view(np.uint16))} groups"
    assert np.array_equal(z.view(np.uint16), z_ref.view(np.uint16)), "zero points differ"
    assert np.array_equal(q, q_ref), f"codes differ at {np.sum(q != q_ref)} weights"


CASES = [
    # n, k, group, widths, lambdas
    (64, 256, 64, [3, 4, 8], [1.0, 1.0, 1.0]),
    (37, 512, 128, [2, 4, 8], [1.0, 0.1, 0.1]),
    (5, 1024, 256, [2, 3, 4, 6, 8], [0.5, 0.25, 0.125, 1.0, 2.0]),
    (16, 2048, 1024, [4, 8], [1.0, 0.3]),
    (3, 64, 64, [8], [1.0]),
    (9, 192, 64, [2], [1.0]),
]


@pytest.mark.parametrize("rule", [O.PREFIX, O.ROUND, O.EXTRA])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}g{c[2]}r{''.join(map(str, c[3]))}")
def test_produce_bitexact(mq, case, rule):
    n, k, group, widths, lams = case
    w = synth.gaussian_weights(synth.rng_for(41, n, k), n, k, outlier_frac=5e-3)
    got, ref = produce_both(mq, w, group, widths, lams, rule)
    assert_same(got, ref)


@pytest.mark.parametrize("n_grid,grid_den", [(1, 1), (1, 100), (17, 40), (100, 100), (256, 256)])
def test_produce_grids(mq, n_grid, grid_den):
    w = synth.gaussian_weights(synth.rng_for(42, n_grid), 24, 512, outlier_frac=1e-2)
    got, ref = produce_both(mq, w, 128, [3, 4, 8], [1.0, 1.0, 1.0], O.PREFIX, n_grid, grid_den)
    assert_same(got, ref)


def test_produce_degenerate_groups(mq):
    w = synth.gaussian_weights(synth.rng_for(43, 0), 8, 512, outlier_frac=0.0)
    w[0, :64] = 0.0                              # all zero: scale 1, zero 0
    w[1, 64:128] = np.float32(0.0125)            # constant positive
    w[2, 128:192] = np.float32(-0.03)            # constant negative
    w[3, 192:256] = np.float32(1e-30)            # range far below the fp16 scale range
    w[4, 256:320] = -np.abs(w[4, 256:320])       # all negative
    w[5, 320:384] *= 1000.0                      # wide range
    w[6, 384:448] = np.float32(2.0 ** -140)      # fp32 denormals
    w[7, ::7] *= 40.0                            # heavy outliers across groups
    for rule in (O.PREFIX, O.ROUND, O.EXTRA):
        got, ref = produce_both(mq, w, 64, [2, 3, 8], [1.0, 0.5, 1.0], rule)
        assert_same(got, ref)
    assert got[1][0, 0] == 1 and got[2][0, 0] == 0


def test_produce_full_matrix_sampled_rows(mq):
    """Llama-3.1-8B gate projection (14336 x 4096, group 128) with MatGPTQ's
    target set {3, 4, 8}: the whole matrix on the GPU, 24 sampled rows of
    every region (first, ragged last block of the search, random) recomputed
    by the oracle row by row (rows are independent)."""
    n, k, group = 14336, 4096, 128
    widths, lams = [3, 4, 8], [1.0, 1.0, 1.0]
    wt = torch.empty((n, k), dtype=torch.float32, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(44)
    wt.normal_(0.0, 0.02, generator=g)
    idx = torch.randint(0, n * k, (int(1e-3 * n * k),), generator=g, device=DEV)
    wt.view(-1)[idx] *= 10.0
    print("[producer] full 14336x4096 group 128 widths {3,4,8}", flush=True)
    q, s, z = mq.produce_parent(wt, group, widths, lams, "prefix")
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, n - 2, n - 1], np.random.default_rng(44).integers(0, n, 20)]))
    w_rows = wt[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    q_ref, s_ref, z_ref = P.produce_parent(w_rows, group, widths, lams, O.PREFIX)
    rows_t = torch.from_numpy(rows).to(DEV)
    assert_same((q[rows_t].cpu().numpy(), s[rows_t].cpu().numpy(), z[rows_t].cpu().numpy()),
                (q_ref, s_ref, z_ref))


@pytest.mark.parametrize("rule", [O.PREFIX, O.ROUND])
def test_produced_parent_serves_every_width(mq, rule):
    """Produce -> pack -> layer at every width of the target set, against the
    oracle's layer on the oracle-produced parent."""
    n, k, group = 256, 1024, 128
    widths, lams = [2, 4, 8], [1.0, 0.1, 0.1]
    w = synth.gaussian_weights(synth.rng_for(45, 0), n, k, outlier_frac=1e-3)
    got, ref = produce_both(mq, w, group, widths, lams, rule)
    assert_same(got, ref)
    q_ref, s_ref, z_ref = ref
    packed = mq.pack_parent(torch.from_numpy(got[0]).to(DEV))
    x = synth.activations(synth.rng_for(45, 1), 3, k, "f16")
    for r in widths:
        y = mq.linear(x.to(DEV), packed, r, rule, group, torch.from_numpy(got[1]).to(DEV),
                      torch.from_numpy(got[2]).to(DEV))
        w64 = O.dequant(q_ref, s_ref, z_ref, r, rule, group)
        x64 = x.double().numpy()
        err = O.normalized_error(y.float().cpu().numpy(), x64 @ w64.T, x64, w64)
        assert err <= 2e-3, (r, err)
