"""HIP path vs the CPU oracle, through the C ABI.

Sliced codes and dequantized weights must match bit for bit; Y must be within
max |dY| / (||X[m,:]|| ||w_hat[n,:]||) <= 2e-3 of the fp64 oracle.  Small
shapes compare every output; the full workload shapes compare sampled output
rows (the oracle dequantizes only those rows)."""
import numpy as np
import pytest
import torch

from oracle import mq_oracle as O
from nested_integer_weight_amd import synth

pytestmark = pytest.mark.gpu

TOL = 2e-3
WIDTHS = [2, 3, 4, 6, 8]
RULES = [O.PREFIX, O.ROUND]
DEV = "cuda:0"


@pytest.fixture(scope="module")
def mq():
    from nested_integer_weight_amd import mq as _mq
    return _mq


def to_dev(lay):
    q = torch.from_numpy(lay.q).to(DEV)
    s = torch.from_numpy(lay.scales).to(DEV)
    z = torch.from_numpy(lay.zeros).to(DEV)
    return q, s, z


def sample_rows(n, count=48, seed=0):
    rng = np.random.default_rng(seed)
    base = {0, 1, n // 2, n - 1}
    base.update(rng.choice(n, size=min(count, n), replace=False).tolist())
    return np.array(sorted(base))


def check_y(y_gpu, lay, x_cpu, r, rule, rows=None, tol=TOL):
    x64 = x_cpu.double().numpy()
    rows = np.arange(lay.n) if rows is None else rows
    w64 = O.dequant(lay.q[rows], lay.scales[rows], lay.zeros[rows], r, rule, lay.group)
    y_ref = x64 @ w64.T
    y = y_gpu.float().cpu().numpy().astype(np.float64)[:, rows]
    assert np.all(np.isfinite(y))
    err = O.normalized_error(y, y_ref, x64, w64)
    assert err <= tol, f"normalized error {err:.3e}"
    return err


# ---------------------------------------------------------------------------
# bit-exact slices and dequantized weights
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def sweep(mq):
    lay = synth.all_codes_layer(96, 1024, 128)
    q, s, z = to_dev(lay)
    return lay, mq.pack_parent(q), s, z


@pytest.fixture(scope="module")
def cfg1(mq):
    lay = synth.make_layer(cfg_id=1, tensor_id=0, n=512, k=512, m=1, group=64, x_dtype="f16")
    q, s, z = to_dev(lay)
    return lay, mq.pack_parent(q), s, z


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("r", WIDTHS)
def test_slice_codes_bitexact(mq, sweep, cfg1, r, rule):
    for lay, pk, _, _ in (sweep, cfg1):
        got = mq.slice_codes(pk, r, rule).cpu().numpy()
        np.testing.assert_array_equal(got, O.slice_code(lay.q, r, rule).astype(np.uint8))
        # only the planes this width needs resident: same codes
        got_t = mq.slice_codes(pk.truncated(r, rule), r, rule).cpu().numpy()
        np.testing.assert_array_equal(got_t, got)


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("r", WIDTHS)
def test_dequant_bitexact(mq, sweep, r, rule):
    lay, pk, s, z = sweep
    w64 = O.dequant(lay.q, lay.scales, lay.zeros, r, rule, lay.group)
    f32 = mq.dequant(pk, r, rule, lay.group, s, z, torch.float32).cpu().numpy()
    np.testing.assert_array_equal(f32.view(np.uint32), O.export_f32(w64).view(np.uint32))
    f16 = mq.dequant(pk, r, rule, lay.group, s, z, torch.float16).cpu().numpy()
    np.testing.assert_array_equal(f16.view(np.uint16), O.export_f16(w64).view(np.uint16))
    b16 = mq.dequant(pk, r, rule, lay.group, s, z, torch.bfloat16).cpu().view(torch.int16).numpy()
    np.testing.assert_array_equal(b16.view(np.uint16), O.export_bf16_bits(w64))


def test_pack_roundtrip_full_width(mq, cfg1):
    lay, pk, _, _ = cfg1
    np.testing.assert_array_equal(mq.slice_codes(pk, 8, O.PREFIX).cpu().numpy(), lay.q)


# ---------------------------------------------------------------------------
# the layer
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("r", WIDTHS)
def test_linear_512_m1(mq, cfg1, r, rule):
    # K = N = 512, M = 1, g = 64, fp16 X ~ N(0,1), both rules
    lay, pk, s, z = cfg1
    x = lay.x.to(DEV)
    y = mq.linear(x, pk, r, rule, lay.group, s, z)
    check_y(y, lay, lay.x, r, rule)


SHAPES = [
    # m, n, k, group, dtype
    (1, 1, 64, 64, "f16"),
    (1, 7, 192, 64, "bf16"),
    (2, 33, 256, 128, "f16"),
    (3, 100, 640, 128, "f16"),
    (4, 65, 4096, 128, "f16"),
    (1, 96, 14336, 128, "f16"),
    (1, 40, 20480, 128, "f16"),     # k beyond the register GEMV: MFMA path at m = 1
    (1, 33, 16384, 128, "bf16"),    # k at the register GEMV's limit (four waves per row)
    (3, 40, 512, 512, "f16"),       # one quantization group per row
    (24, 72, 1024, 1024, "f16"),    # skinny with one group per row
    (2, 50, 1024, 64, "bf16"),
    (5, 300, 640, 128, "f16"),
    (8, 257, 1024, 64, "f16"),
    (17, 129, 2048, 128, "bf16"),
    (63, 64, 512, 64, "f16"),
    (4, 70, 768, 64, "bf16"),       # skinny MFMA path: bf16 m = 4, three k rounds
    (16, 1, 256, 64, "f16"),        # skinny: a single output column and round
    (33, 200, 1536, 256, "f16"),    # skinny: three m tiles, group 256
    (49, 130, 2304, 128, "bf16"),   # skinny: four m tiles, nine rounds split nine ways
    (64, 17, 4352, 128, "f16"),     # skinny: seventeen rounds, ragged n
    (12, 384, 3584, 128, "f16"),    # skinny: fourteen rounds split seven ways
    (5, 14400, 512, 64, "f16"),     # skinny with 64-row workgroups (wide n, no k split)
    (20, 14337, 256, 128, "bf16"),  # skinny 64-row workgroups, two m tiles, one-row tail block
    (20, 14400, 768, 64, "bf16"),   # skinny, two k teams per workgroup: 2 + 1 rounds
    (33, 14336, 1280, 128, "f16"),  # skinny, two k teams: 3 + 2 rounds, three m tiles
    (40, 8192, 3840, 128, "f16"),   # skinny, two k teams under a four-way k split (2 + 2, last 2 + 1)
    (9, 14336, 1024, 128, "f16"),   # skinny, 128-code runs per lane: two rounds of 512
    (24, 14336, 1536, 128, "f16"),  # skinny, 128-code runs (r >= 4), two k teams: 2 + 1 rounds
    (32, 14352, 512, 128, "bf16"),  # skinny, 128-code runs (r >= 4), two k teams: 1 + 0 rounds, ragged n
    (40, 14401, 2560, 256, "bf16"), # skinny, 128-code runs, three m tiles, one X buffer per team, group 256, ragged n
    (48, 14336, 1536, 128, "f16"),  # skinny, 128-code runs, three m tiles, one X buffer per team: 2 + 1 rounds
    (65, 300, 768, 64, "bf16"),
    (257, 300, 512, 128, "bf16"),
    (300, 448, 1024, 128, "bf16"),  # prefill tile with split k
    (257, 672, 2048, 64, "f16"),    # prefill tile, ragged m, group 64
    (300, 520, 1024, 128, "f16"),
]


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("r", [2, 3, 8])
@pytest.mark.parametrize("m,n,k,group,dt", SHAPES, ids=lambda v: str(v))
def test_linear_shapes(mq, m, n, k, group, dt, r, rule):
    lay = synth.make_layer(cfg_id=6, tensor_id=n * 7 + m, n=n, k=k, m=m, group=group, x_dtype=dt)
    q, s, z = to_dev(lay)
    pk = mq.pack_parent(q)
    x = lay.x.to(DEV)
    y = mq.linear(x, pk, r, rule, group, s, z)
    assert y.dtype == x.dtype and y.shape == (m, n)
    check_y(y, lay, lay.x, r, rule)


def test_linear_m0_is_noop(mq, cfg1):
    lay, pk, s, z = cfg1
    x = torch.empty((0, lay.k), dtype=torch.float16, device=DEV)
    y = mq.linear(x, pk, 4, O.PREFIX, lay.group, s, z)
    assert y.shape == (0, lay.n)


def test_determinism_and_split_k(mq):
    lay = synth.make_layer(cfg_id=6, tensor_id=999, n=512, k=4096, m=24, group=128, x_dtype="f16")
    q, s, z = to_dev(lay)
    pk = mq.pack_parent(q)
    x = lay.x.to(DEV)
    y1 = mq.linear(x, pk, 4, O.PREFIX, 128, s, z)
    y2 = mq.linear(x, pk, 4, O.PREFIX, 128, s, z)
    assert torch.equal(y1, y2)
    y3 = mq.linear(x, pk, 4, O.PREFIX, 128, s, z, workspace=None)  # no split-k
    check_y(y1, lay, lay.x, 4, O.PREFIX)
    check_y(y3, lay, lay.x, 4, O.PREFIX)
    assert mq.workspace_bytes(24, 512, 4096) > 0


def test_mixed_equals_single_calls(mq):
    calls, lays = [], []
    for i, (r, m, dt) in enumerate([(2, 1, "f16"), (3, 1, "f16"), (4, 8, "f16"), (8, 40, "bf16"), (2, 200, "bf16")]):
        lay = synth.make_layer(cfg_id=5, tensor_id=100 + i, n=320, k=1024, m=m, group=128, x_dtype=dt)
        q, s, z = to_dev(lay)
        calls.append(mq.Call(x=lay.x.to(DEV), packed=mq.pack_parent(q), r=r, rule=O.PREFIX, group=128,
                             scales=s, zeros=z))
        lays.append(lay)
    outs = mq.linear_mixed(calls)
    for c, lay, y in zip(calls, lays, outs):
        single = mq.linear(c.x, c.packed, c.r, c.rule, c.group, c.scales, c.zeros)
        assert torch.equal(single, y)
        check_y(y, lay, lay.x, c.r, c.rule)


@pytest.mark.parametrize("m,dt,r,rule,group", [(1, "f16", 2, O.PREFIX, 128), (3, "f16", 3, O.ROUND, 64),
                                                (1, "bf16", 8, O.PREFIX, 128), (2, "f16", 6, O.PREFIX, 256)])
def test_mixed_batches_independent_gemv_calls(mq, m, dt, r, rule, group):
    # five independent calls of one shape class with ragged n: the library runs
    # the first four in one launch and the fifth alone; each result must equal
    # its single call bit for bit and the oracle within tolerance
    calls, lays = [], []
    for i, n in enumerate((1, 70, 333, 8, 1025)):
        lay = synth.make_layer(cfg_id=5, tensor_id=300 + 10 * i + r, n=n, k=1024, m=m, group=group, x_dtype=dt)
        q, s, z = to_dev(lay)
        calls.append(mq.Call(x=lay.x.to(DEV), packed=mq.pack_parent(q), r=r, rule=rule, group=group,
                             scales=s, zeros=z))
        lays.append(lay)
    outs = mq.linear_mixed(calls)
    for c, lay, y in zip(calls, lays, outs):
        single = mq.linear(c.x, c.packed, c.r, c.rule, c.group, c.scales, c.zeros)
        assert torch.equal(single, y)
        check_y(y, lay, lay.x, c.r, c.rule)


def test_mixed_dependent_gemv_calls_keep_order(mq):
    # same shape class throughout (m = 1, k = n = 512), but B reads A's output,
    # C overwrites A's output and D is independent: the result must be that of
    # the calls issued one by one
    k = 512
    lays, packs = [], []
    for i in range(4):
        lay = synth.make_layer(cfg_id=5, tensor_id=400 + i, n=k, k=k, m=1, group=128, x_dtype="f16")
        q, s, z = to_dev(lay)
        lays.append(lay)
        packs.append((mq.pack_parent(q), s, z))
    x0 = lays[0].x.to(DEV)
    x3 = lays[3].x.to(DEV)
    ya = torch.empty((1, k), dtype=torch.float16, device=DEV)
    yb = torch.empty((1, k), dtype=torch.float16, device=DEV)
    yd = torch.empty((1, k), dtype=torch.float16, device=DEV)

    def calls():
        return [mq.Call(x=x0, packed=packs[0][0], r=4, rule=O.PREFIX, group=128, scales=packs[0][1],
                        zeros=packs[0][2], out=ya),
                mq.Call(x=ya, packed=packs[1][0], r=4, rule=O.PREFIX, group=128, scales=packs[1][1],
                        zeros=packs[1][2], out=yb),
                mq.Call(x=x3, packed=packs[2][0], r=4, rule=O.PREFIX, group=128, scales=packs[2][1],
                        zeros=packs[2][2], out=ya),
                mq.Call(x=x3, packed=packs[3][0], r=4, rule=O.PREFIX, group=128, scales=packs[3][1],
                        zeros=packs[3][2], out=yd)]

    mq.linear_mixed(calls())
    got = [ya.clone(), yb.clone(), yd.clone()]
    for c in calls():
        mq.linear(c.x, c.packed, c.r, c.rule, c.group, c.scales, c.zeros, out=c.out)
    assert torch.equal(got[0], ya) and torch.equal(got[1], yb) and torch.equal(got[2], yd)


# ---------------------------------------------------------------------------
# full workload shapes, sampled rows
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def llama_ffn(mq):
    out = []
    for tid, (name, n, k) in enumerate(synth.LLAMA8B_FFN):
        lay = synth.make_layer(cfg_id=2, tensor_id=tid, n=n, k=k, m=0, group=128, outlier_frac=1e-3)
        q, s, z = to_dev(lay)
        out.append((name, lay, mq.pack_parent(q), s, z))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("r", WIDTHS)
def test_llama_ffn_decode_m1(mq, llama_ffn, r):
    for name, lay, pk, s, z in llama_ffn:
        x = synth.activations(synth.rng_for(2, 10 + r), 1, lay.k, "f16")
        y = mq.linear(x.to(DEV), pk.truncated(r), r, O.PREFIX, 128, s, z)
        check_y(y, lay, x, r, O.PREFIX, rows=sample_rows(lay.n))


@pytest.mark.parametrize("m", [8, 16, 32, 64])
def test_llama_ffn_skinny(mq, llama_ffn, m):
    for r in (2, 3, 4, 8):
        for name, lay, pk, s, z in llama_ffn:
            x = synth.activations(synth.rng_for(3, m, r), m, lay.k, "f16")
            y = mq.linear(x.to(DEV), pk, r, O.PREFIX, 128, s, z)
            check_y(y, lay, x, r, O.PREFIX, rows=sample_rows(lay.n, 24))


@pytest.mark.parametrize("r", [2, 3, 6])
def test_llama_ffn_decode_m1_round_rule(mq, llama_ffn, r):
    # the rounded slice at the full decode shapes (it reads one more plane)
    for name, lay, pk, s, z in llama_ffn:
        x = synth.activations(synth.rng_for(2, 20 + r), 1, lay.k, "f16")
        y = mq.linear(x.to(DEV), pk, r, O.ROUND, 128, s, z)
        check_y(y, lay, x, r, O.ROUND, rows=sample_rows(lay.n))


@pytest.mark.parametrize("m", [1, 8, 40])
def test_llama_ffn_bf16_decode(mq, llama_ffn, m):
    # bf16 activations at the full shapes: GEMV at m = 1, skinny above
    for r in (2, 4, 8):
        for name, lay, pk, s, z in llama_ffn:
            x = synth.activations(synth.rng_for(3, 100 + m, r), m, lay.k, "bf16")
            y = mq.linear(x.to(DEV), pk, r, O.PREFIX, 128, s, z)
            check_y(y, lay, x, r, O.PREFIX, rows=sample_rows(lay.n, 24))


@pytest.mark.parametrize("r", [2, 4, 8])
def test_llama_ffn_prefill_2048(mq, llama_ffn, r):
    for name, lay, pk, s, z in llama_ffn:
        x = synth.activations(synth.rng_for(4, r), 2048, lay.k, "bf16")
        y = mq.linear(x.to(DEV), pk, r, O.PREFIX, 128, s, z)
        check_y(y, lay, x, r, O.PREFIX, rows=sample_rows(lay.n, 16))


@pytest.mark.parametrize("m,dt", [(1, "f16"), (256, "bf16")])
def test_gemma_mixnmatch_blocks(mq, m, dt):
    widths = synth.mixnmatch_widths()
    calls, meta = [], []
    for blk in range(3):  # three of the 42 blocks: one of each width in the seeded order
        r = widths[blk]
        for tid, (name, n, k) in enumerate(synth.GEMMA9B_FFN):
            lay = synth.make_layer(cfg_id=5, tensor_id=tid, n=n, k=k, m=0, group=128, extra=(blk,))
            q, s, z = to_dev(lay)
            x = synth.activations(synth.rng_for(5, 50 + tid, blk, m), m, k, dt)
            calls.append(mq.Call(x=x.to(DEV), packed=mq.pack_parent(q), r=r, rule=O.PREFIX, group=128,
                                 scales=s, zeros=z))
            meta.append((lay, x, r))
    outs = mq.linear_mixed(calls)
    for (lay, x, r), y in zip(meta, outs):
        check_y(y, lay, x, r, O.PREFIX, rows=sample_rows(lay.n, 16))


def test_graph_replay_matches_eager(mq):
    # the serving form: calls captured in a HIP graph (GEMV, skinny with split-k,
    # GEMM with split-k) replay bit for bit like the eager calls, replay after
    # replay, with eager work and synchronisation in between
    calls = []
    for i, (r, m, dt, n, k) in enumerate([(2, 1, "f16", 512, 4096), (4, 16, "f16", 640, 4096),
                                          (8, 40, "bf16", 384, 2048), (3, 300, "bf16", 520, 1024)]):
        lay = synth.make_layer(cfg_id=7, tensor_id=i, n=n, k=k, m=m, group=128, x_dtype=dt)
        q, s, z = to_dev(lay)
        x = lay.x.to(DEV)
        calls.append(mq.Call(x=x, packed=mq.pack_parent(q), r=r, rule=O.PREFIX, group=128, scales=s, zeros=z,
                             out=torch.empty((m, n), dtype=x.dtype, device=DEV)))
    eager = [y.clone() for y in mq.linear_mixed(calls)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mq.linear_mixed(calls)
    for rep in range(3):
        for c in calls:
            c.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        for c, y0 in zip(calls, eager):
            assert torch.equal(c.out, y0), f"replay {rep} differs"
        mq.linear_mixed(calls[:1])  # eager work between replays
        torch.cuda.synchronize()
