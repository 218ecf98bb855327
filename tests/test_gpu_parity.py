"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Codes, block scales, tensor scales and dequantized values must be
bit-identical; statistics agree within 1e-6 relative with an absolute floor
of 1e-6 * mean|v| (binary64 sums in a different order).
"""
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

E1M2, INT4, E2M1, E2M1C = 0, 1, 2, 3
RTNE, SR = 0, 1
NV16, MX32 = 0, 1
ROW, COL = 0, 1
AUTO, TWO_PASS, SINGLE_PASS = 0, 1, 2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp4_quantization_amd as F
    import oracle
    oracle.lib()
    return torch, F, oracle


@pytest.fixture
def schedule(env):
    """Set the process-wide schedule for one test; restored to AUTO after."""
    _, F, _ = env

    def set_(mode, left_stride=0):
        F.ufp4_set_schedule(mode, left_stride)

    yield set_
    F.ufp4_set_schedule(AUTO, 0)


def to_dev(torch, xb):
    return torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).cuda()


def cfgs(F, orc, grid=E1M2, rounding=RTNE, scaling=NV16, rht=1, rht_seed=0, sr_seed=0):
    return (F.config(grid, rounding, scaling, rht, rht_seed, sr_seed),
            orc.config(grid, rounding, scaling, rht, rht_seed, sr_seed))


def gpu_rowcol(env, xb, fc):
    torch, F, _ = env
    R, C = xb.shape
    x = to_dev(torch, xb)
    row = F.alloc_layout(R, C, fc.scaling)
    col = F.alloc_layout(C, R, fc.scaling)
    ws = F.Workspace(R, C)
    F.ufp4_quantize_rowcol(x, fc, row, col, ws)
    torch.cuda.synchronize()
    return row, col


def gpu_row(env, xb, fc, ld=None):
    torch, F, _ = env
    R, C = xb.shape
    if ld is not None and ld != C:
        buf = np.zeros((R, ld), np.uint16)
        buf[:, :C] = xb
        x = to_dev(torch, buf)[:, :C]
    else:
        x = to_dev(torch, xb)
    row = F.alloc_layout(R, C, fc.scaling)
    ws = F.Workspace(R, C)
    F.ufp4_quantize(x, fc, row, ws)
    torch.cuda.synchronize()
    return row


def assert_layout_equal(q, ref, what):
    c, s, t = ref
    gc, gs, gt = q.codes.cpu().numpy(), q.scales.cpu().numpy(), q.tensor_scale.cpu().numpy()
    if not np.array_equal(gc, c):
        bad = np.argwhere(gc != c)
        raise AssertionError(f"{what}: {len(bad)} code bytes differ, first at {bad[:5].tolist()}")
    if not np.array_equal(gs, s):
        bad = np.argwhere(gs != s)
        raise AssertionError(f"{what}: {len(bad)} scale bytes differ, first at {bad[:5].tolist()}")
    assert gt.view(np.uint32)[: t.size].tolist() == t.view(np.uint32).tolist(), f"{what}: tensor scale"


# ------------------------------------------------------------- rounding hook
@pytest.mark.parametrize("grid", [E1M2, INT4, E2M1, E2M1C])
@pytest.mark.parametrize("rounding", [RTNE, SR])
def test_round_f32_all_bf16_patterns(env, grid, rounding):
    torch, F, orc = env
    say(f"[round_f32] grid={grid} rounding={rounding}")
    y = synth.all_bf16_patterns()
    want = orc.round_f32(y, grid, rounding, sr_seed=5)
    yd = torch.from_numpy(y).cuda()
    codes = torch.empty(y.size, dtype=torch.uint8, device="cuda")
    F.ufp4_round_f32(yd, grid, rounding, 5, codes)
    np.testing.assert_array_equal(codes.cpu().numpy(), want)


def test_round_f32_dense_fp32_sweep(env):
    # every fp32 bit pattern in [0, 8) with a stride, both signs, all grids,
    # both roundings: catches ties and bucket edges beyond bf16 precision
    torch, F, orc = env
    say("[round_f32] fp32 sweep")
    bits = np.arange(0, 0x41000000, 257, dtype=np.uint32)
    y = np.concatenate([bits.view(np.float32), -bits.view(np.float32)])
    yd = torch.from_numpy(y).cuda()
    codes = torch.empty(y.size, dtype=torch.uint8, device="cuda")
    for grid in (E1M2, INT4, E2M1, E2M1C):
        for rounding in (RTNE, SR):
            F.ufp4_round_f32(yd, grid, rounding, 9, codes)
            np.testing.assert_array_equal(codes.cpu().numpy(), orc.round_f32(y, grid, rounding, sr_seed=9))


# -------------------------------------------------------------- tiny config
def test_tiny_config_row(env):
    torch, F, orc = env
    say("[tiny] 256x256 RHT E1M2 RTNE row-wise")
    xb = synth.tiny(0)
    fc, oc = cfgs(F, orc, rht_seed=0)
    assert_layout_equal(gpu_row(env, xb, fc), orc.quantize(xb, oc, ROW), "tiny row")


# ------------------------------------------------ small shapes, all variants
SHAPES = [(384, 320), (160, 512), (32, 2048)]


@pytest.mark.parametrize("sched", [TWO_PASS, SINGLE_PASS])
@pytest.mark.parametrize("grid", [E1M2, INT4, E2M1, E2M1C])
@pytest.mark.parametrize("rounding", [RTNE, SR])
@pytest.mark.parametrize("scaling", [NV16, MX32])
@pytest.mark.parametrize("rht", [1, 0])
def test_rowcol_variants(env, schedule, sched, grid, rounding, scaling, rht):
    # (MX32 has no tensor maximum: both schedules run its one kernel)
    torch, F, orc = env
    schedule(sched)
    for shape in SHAPES:
        R, C = shape
        say(f"[rowcol] {R}x{C} grid={grid} rnd={rounding} scl={scaling} rht={rht} sched={sched}")
        xb = synth.activation(R, C, seed=R + C + grid)
        fc, oc = cfgs(F, orc, grid, rounding, scaling, rht, rht_seed=3, sr_seed=11)
        row, col = gpu_rowcol(env, xb, fc)
        assert_layout_equal(row, orc.quantize(xb, oc, ROW), f"row {shape}")
        assert_layout_equal(col, orc.quantize(xb, oc, COL), f"col {shape}")


@pytest.mark.parametrize("scaling", [NV16, MX32])
def test_row_ragged_rows_and_padded_ld(env, scaling):
    torch, F, orc = env
    for R, C, ld in [(1, 32, 32), (100, 64, 72), (129, 96, 96), (300, 256, 264)]:
        say(f"[row ragged] {R}x{C} ld={ld} scl={scaling}")
        xb = synth.output_grad(R, C, seed=R)
        fc, oc = cfgs(F, orc, E1M2, SR, scaling, 1, rht_seed=1, sr_seed=2)
        assert_layout_equal(gpu_row(env, xb, fc, ld=ld), orc.quantize(xb, oc, ROW), f"row {R}x{C}")


def test_edge_values(env):
    torch, F, orc = env
    R, C = 64, 64
    cases = {
        "zeros": np.zeros((R, C), np.uint16),
        "one_nonzero": np.where(np.arange(R * C).reshape(R, C) == 777, 0x3F80, 0).astype(np.uint16),
        "tiny": synth.f32_to_bf16(np.random.default_rng(1).standard_normal((R, C)).astype(np.float32) * 1e-38),
        "subnormal_bf16": (np.random.default_rng(2).integers(0, 0x80, (R, C)) |
                           (np.random.default_rng(3).integers(0, 2, (R, C)) << 15)).astype(np.uint16),
        "huge": synth.f32_to_bf16(np.random.default_rng(4).standard_normal((R, C)).astype(np.float32) * 1e36),
        "mixed_scale": synth.f32_to_bf16(np.random.default_rng(5).standard_normal((R, C)).astype(np.float32) *
                                         (10.0 ** np.random.default_rng(6).integers(-30, 30, (R, C))).astype(np.float32)),
    }
    for name, xb in cases.items():
        for grid in (E1M2, INT4, E2M1, E2M1C):
            for scaling in (NV16, MX32):
                for rounding in (RTNE, SR):
                    say(f"[edge] {name} grid={grid} scl={scaling} rnd={rounding}")
                    fc, oc = cfgs(F, orc, grid, rounding, scaling, 1, rht_seed=4, sr_seed=4)
                    row, col = gpu_rowcol(env, xb, fc)
                    assert_layout_equal(row, orc.quantize(xb, oc, ROW), f"{name} row")
                    assert_layout_equal(col, orc.quantize(xb, oc, COL), f"{name} col")


def test_e2m1_ties_through_the_packed_conversion(env, schedule):
    # Without the transform, a tensor maximum of 6 * 448 makes the NV16
    # tensor scale 1 and a 6.0 at the start of every 16-long row and column
    # block makes those blocks' scales 1 (the MX32 scale of a 6.0 block is
    # 2^0 as well), so the scaled values are the inputs themselves: exact
    # E2M1 ties (0.25, 0.75, ..., 5) and grid values, rounded to nearest
    # even by the packed hardware conversion.  Both schedules, both layouts.
    torch, F, orc = env
    R, C = 64, 96
    rng = np.random.default_rng(41)
    vals = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 3.0, 4.0, 6.0, 0.0], np.float32)
    x = rng.choice(vals, (R, C)) * rng.choice(np.array([-1.0, 1.0], np.float32), (R, C))
    x[:, ::16] = 6.0
    x[::16, :] = -6.0
    x[0, 0] = 6.0 * 448.0
    xb = synth.f32_to_bf16(x.astype(np.float32))
    assert np.array_equal(synth.bf16_to_f32(xb), x.astype(np.float32))
    for sched in (TWO_PASS, SINGLE_PASS):
        schedule(sched)
        for grid in (E2M1, E1M2):
            for scaling in (NV16, MX32):
                say(f"[e2m1 ties] sched={sched} grid={grid} scl={scaling}")
                fc, oc = cfgs(F, orc, grid, RTNE, scaling, 0, rht_seed=1, sr_seed=1)
                row, col = gpu_rowcol(env, xb, fc)
                assert_layout_equal(row, orc.quantize(xb, oc, ROW), "ties row")
                assert_layout_equal(col, orc.quantize(xb, oc, COL), "ties col")


def nonfinite_input(R, C, seed, inf=True):
    """Normal values with about 1% NaN and (if inf) 1% each of +-inf, bf16."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, C)).astype(np.float32)
    u = rng.random((R, C))
    x[u < 0.01] = np.nan
    if inf:
        x[(u >= 0.01) & (u < 0.02)] = np.inf
        x[(u >= 0.02) & (u < 0.03)] = -np.inf
    return synth.f32_to_bf16(x)


@pytest.mark.parametrize("rht", [0, 1])
@pytest.mark.parametrize("sched", [TWO_PASS, SINGLE_PASS])
def test_nonfinite_inputs(env, schedule, rht, sched):
    # NaN codes to 0 and is left out of every maximum; +-inf saturates (and,
    # through the transform, turns its block into NaN and inf values); with
    # inf present the tensor scale is inf.  Both with and without inf.
    torch, F, orc = env
    schedule(sched)
    R, C = 96, 160
    for inf in (False, True):
        xb = nonfinite_input(R, C, seed=31 + rht, inf=inf)
        for grid in (E1M2, INT4, E2M1, E2M1C):
            for scaling in (NV16, MX32):
                for rounding in (RTNE, SR):
                    say(f"[nonfinite] inf={inf} rht={rht} sched={sched} grid={grid} scl={scaling} rnd={rounding}")
                    fc, oc = cfgs(F, orc, grid, rounding, scaling, rht, rht_seed=5, sr_seed=5)
                    row, col = gpu_rowcol(env, xb, fc)
                    assert_layout_equal(row, orc.quantize(xb, oc, ROW), "nonfinite row")
                    assert_layout_equal(col, orc.quantize(xb, oc, COL), "nonfinite col")


def test_empty_tensor(env):
    torch, F, orc = env
    fc, _ = cfgs(F, orc)
    x = torch.zeros((0, 64), dtype=torch.int16, device="cuda")
    row = F.alloc_layout(0, 64, NV16)
    F.ufp4_quantize(x, fc, row, F.Workspace(16, 64))
    torch.cuda.synchronize()
    assert row.tensor_scale.item() == 1.0


def test_deterministic_repeat(env):
    torch, F, orc = env
    xb = synth.output_grad(256, 512, seed=8)
    fc, _ = cfgs(F, orc, E1M2, SR, NV16, 1, 1, 1)
    a = gpu_rowcol(env, xb, fc)
    b = gpu_rowcol(env, xb, fc)
    for qa, qb in zip(a, b):
        assert torch.equal(qa.codes, qb.codes) and torch.equal(qa.scales, qb.scales)


def test_identical_bytes_across_schedules_and_work_distributions(env, schedule):
    # the kernels' tile size is fixed by the lane geometry, so the launch
    # variants are the schedules and the assignment of tiles to workgroups:
    # two passes, one pass, one pass with tiles left to other workgroups
    # (strides 2, 3, 7), the no-allocation entry point, delayed scaling under
    # the tensor's own maxima, and a grouped call with one segment all give
    # the same bytes, each repeated, with stochastic rounding (whose words
    # are tied to output positions) and the transform on
    torch, F, orc = env
    R, C = 640, 1280
    xb = synth.output_grad(R, C, seed=61)
    fc, _ = cfgs(F, orc, E1M2, SR, NV16, 1, 9, 9)
    x = to_dev(torch, xb)

    def outs():
        return F.alloc_layout(R, C, NV16), F.alloc_layout(C, R, NV16)

    def grab(pair):
        torch.cuda.synchronize()
        return [t.clone() for q in pair for t in (q.codes, q.scales, q.tensor_scale)]

    results = {}
    ws = F.Workspace(R, C)
    for name, mode, stride in (("two_pass", TWO_PASS, 0), ("single", SINGLE_PASS, 0), ("left2", SINGLE_PASS, 2),
                               ("left3", SINGLE_PASS, 3), ("left7", SINGLE_PASS, 7)):
        schedule(mode, stride)
        for rep in range(2):
            pair = outs()
            F.ufp4_quantize_rowcol(x, fc, *pair, ws)
            results[f"{name}.{rep}"] = grab(pair)
    schedule(AUTO, 0)
    for rep in range(2):
        pair = outs()
        F.ufp4_quantize_rowcol_noalloc(x, fc, *pair)
        results[f"noalloc.{rep}"] = grab(pair)
    n = F.ufp4_amax_tiles(R, C)
    a1 = torch.zeros((n, 2), dtype=torch.float32, device="cuda")
    a2 = torch.zeros((n, 2), dtype=torch.float32, device="cuda")
    F.ufp4_quantize_delayed(x, fc, torch.ones((1, 2), dtype=torch.float32, device="cuda"), a1, *outs())
    pair = outs()
    F.ufp4_quantize_delayed(x, fc, a1, a2, *pair)
    results["delayed_own"] = grab(pair)
    pair = outs()
    F.ufp4_quantize_grouped(x, torch.tensor([0, R], dtype=torch.int64, device="cuda"), R, fc, *pair,
                            F.Workspace(R, C, 1))
    results["grouped_one_segment"] = grab(pair)
    ref = results.pop("two_pass.0")
    for name, got in results.items():
        for i, (u, v) in enumerate(zip(ref, got)):
            assert torch.equal(u, v), f"{name}: output {i} differs from the two-pass call"


@pytest.mark.parametrize("sched", [TWO_PASS, SINGLE_PASS])
def test_timing_hook_matches_plain_call(env, schedule, sched):
    torch, F, orc = env
    schedule(sched)
    xb = synth.activation(384, 512, seed=9)
    fc, oc = cfgs(F, orc, E1M2, RTNE, NV16, 1, 9, 9)
    x = to_dev(torch, xb)
    row, col = F.alloc_layout(384, 512, NV16), F.alloc_layout(512, 384, NV16)
    ms_a, ms_q = F.ufp4_time_rowcol(x, fc, row, col, F.Workspace(384, 512))
    # the single pass has no separate maxima kernel: its time is reported as 0
    assert ms_q > 0.0 and (ms_a > 0.0 if sched == TWO_PASS else ms_a == 0.0)
    for name, qt, layout in (("row", row, ROW), ("col", col, COL)):
        c, s_, t = orc.quantize(xb, oc, layout)
        assert np.array_equal(qt.codes.cpu().numpy(), c), name
        assert np.array_equal(qt.scales.cpu().numpy(), s_), name
        assert qt.tensor_scale.cpu().numpy().view(np.uint32)[0] == t.view(np.uint32)[0], name


# ------------------------------------------------------------------ delayed
def gpu_delayed(env, xb, fc, amax_in, col=True):
    """One delayed call; amax_in: float32 array of (row, col) pairs, or a
    device tensor.  Returns (row, col, tile maxima as numpy [n, 2])."""
    torch, F, _ = env
    R, C = xb.shape
    x = to_dev(torch, xb)
    row = F.alloc_layout(R, C, NV16)
    colq = F.alloc_layout(C, R, NV16) if col else None
    if isinstance(amax_in, torch.Tensor):
        a_in = amax_in
    else:
        a_in = torch.from_numpy(np.asarray(amax_in, np.float32).reshape(-1, 2).copy()).cuda()
    n = F.ufp4_amax_tiles(R, C)
    a_out = torch.full((n, 2), -1.0, dtype=torch.float32, device="cuda")
    F.ufp4_quantize_delayed(x, fc, a_in, a_out, row, colq)
    torch.cuda.synchronize()
    return row, colq, a_out


def own_maxima(orc, xb, oc):
    r = orc.quantize_given_amax(xb, oc, ROW, 1.0)[3]
    c = orc.quantize_given_amax(xb, oc, COL, 1.0)[3]
    return np.float32(r), np.float32(c)


@pytest.mark.parametrize("grid", [E1M2, INT4, E2M1, E2M1C])
@pytest.mark.parametrize("rounding", [RTNE, SR])
@pytest.mark.parametrize("rht", [1, 0])
def test_delayed_matches_oracle(env, grid, rounding, rht):
    # provided maxima at, below (saturating) and above the tensor's own
    torch, F, orc = env
    for R, C in ((384, 320), (160, 512)):
        xb = synth.activation(R, C, seed=R + grid + 7)
        fc, oc = cfgs(F, orc, grid, rounding, NV16, rht, 3, 11)
        mr, mc = own_maxima(orc, xb, oc)
        for factor in (1.0, 0.25, 3.0):
            gr, gc = np.float32(mr * np.float32(factor)), np.float32(mc * np.float32(factor))
            say(f"[delayed] {R}x{C} grid={grid} rnd={rounding} rht={rht} x{factor}")
            row, col, a_out = gpu_delayed(env, xb, fc, [gr, gc])
            want_r = orc.quantize_given_amax(xb, oc, ROW, float(gr))
            want_c = orc.quantize_given_amax(xb, oc, COL, float(gc))
            assert_layout_equal(row, want_r[:3], f"row x{factor}")
            assert_layout_equal(col, want_c[:3], f"col x{factor}")
            if factor == 1.0:
                assert_layout_equal(row, orc.quantize(xb, oc, ROW), "row = exact path")
                assert_layout_equal(col, orc.quantize(xb, oc, COL), "col = exact path")
            t = a_out.cpu().numpy()
            assert (t >= 0).all(), "every tile maximum written"
            assert t[:, 0].max() == mr and t[:, 1].max() == mc


def test_delayed_chain_reaches_exact_path(env):
    # a first call with an arbitrary provided maximum; its tile maxima, passed
    # as they are, make the second call the exact (own-maximum) quantization
    torch, F, orc = env
    R, C = 1040, 1024
    xb = synth.activation(R, C, seed=50)
    fc, oc = cfgs(F, orc, E1M2, RTNE, NV16, 1, 4, 4)
    _, _, a1 = gpu_delayed(env, xb, fc, [1.0, 1.0])
    row, col, a2 = gpu_delayed(env, xb, fc, a1)
    assert_layout_equal(row, orc.quantize(xb, oc, ROW), "row")
    assert_layout_equal(col, orc.quantize(xb, oc, COL), "col")
    assert torch.equal(a1, a2)


def test_delayed_row_only_nonfinite_and_many_entries(env):
    torch, F, orc = env
    R, C = 200, 256
    xb = synth.output_grad(R, C, seed=51)
    fc, oc = cfgs(F, orc, E1M2, SR, NV16, 1, 6, 6)
    # entries that are not positive finite numbers count as zero: S_t = 1
    row, _, _ = gpu_delayed(env, xb, fc, [np.nan, np.inf, -1.0, 0.0, -np.inf, np.nan], col=False)
    assert_layout_equal(row, orc.quantize_given_amax(xb, oc, ROW, 0.0)[:3], "non-finite")
    # 700 entries (more than one per thread); the largest row-wise entry decides
    mr = np.float32(orc.quantize_given_amax(xb, oc, ROW, 1.0)[3])  # (200 rows: no column layout)
    ent = np.zeros((700, 2), np.float32)
    ent[:, 0] = np.linspace(0, 0.5, 700, dtype=np.float32) * mr
    ent[650, 0] = mr * np.float32(0.75)
    ent[:, 1] = np.nan
    row, _, a_out = gpu_delayed(env, xb, fc, ent, col=False)
    assert_layout_equal(row, orc.quantize_given_amax(xb, oc, ROW, float(ent[:, 0].max()))[:3], "700 entries")
    t = a_out.cpu().numpy()
    assert t[:, 0].max() == mr and (t[:, 1] == 0).all()


# ------------------------------------------------------------ consumer GEMM
def upload(torch, F, q, rows, cols, scaling=NV16):
    """An oracle-quantized row-wise layout as a device QTensor."""
    qt = F.alloc_layout(rows, cols, scaling)
    qt.codes.copy_(torch.from_numpy(np.ascontiguousarray(q[0])))
    qt.scales.copy_(torch.from_numpy(np.ascontiguousarray(q[1])))
    qt.tensor_scale.copy_(torch.from_numpy(np.ascontiguousarray(q[2])))
    return qt


@pytest.mark.parametrize("scaling", [NV16, MX32])
@pytest.mark.parametrize("grid", [E1M2, INT4, E2M1, E2M1C])
def test_gemm_matches_oracle_reference(env, grid, scaling):
    # operands quantized by the oracle; the GEMM against the float64 product
    # of the oracle's dequantized operands, within the fp32 accumulation bound
    torch, F, orc = env
    for M, N, K in ((256, 384, 512), (130, 70, 96), (1, 1, 32), (300, 129, 2048), (257, 513, 160)):
        say(f"[gemm] grid={grid} scaling={scaling} {M}x{N}x{K}")
        fc, oc = cfgs(F, orc, grid, RTNE, scaling, 1, 7, 7)
        a = orc.quantize(synth.activation(M, K, seed=M + K), oc, ROW)
        b = orc.quantize(synth.weight(N, K, seed=N + K), oc, ROW)
        ref, mag = orc.gemm_nt_reference(a, b, oc, M, N, K)
        c = torch.full((M, N + 3), np.nan, dtype=torch.float32, device="cuda")[:, :N]
        F.ufp4_gemm_nt(fc, upload(torch, F, a, M, K, scaling), upload(torch, F, b, N, K, scaling), M, N, K, c)
        torch.cuda.synchronize()
        got = c.cpu().numpy().astype(np.float64)
        bound = (K + 4) * 2.0 ** -24 * mag + 1e-30
        err = np.abs(got - ref)
        assert (err <= bound).all(), f"max err/bound {float((err / bound).max()):.3g}"


def test_gemm_exact_on_exactly_representable_products(env):
    # integer-valued operands (INT4 codes, unit block scales, unit tensor
    # scales) with small sums: every partial sum is an integer below 2^24,
    # so the fp32 MFMA result is exact
    torch, F, orc = env
    rng = np.random.default_rng(40)
    M, N, K = 64, 96, 256
    fc, oc = cfgs(F, orc, INT4, RTNE, NV16, 0, 0, 0)

    def layout(rows):
        k = rng.integers(-7, 8, size=(rows, K))
        nib = (k & 15).astype(np.uint8)
        codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
        scales = np.full((rows, K // 16), 0x38, np.uint8)  # E4M3 1.0
        return (codes, scales, np.ones(1, np.float32)), k.astype(np.float64)

    (a, ka), (b, kb) = layout(M), layout(N)
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    F.ufp4_gemm_nt(fc, upload(torch, F, a, M, K), upload(torch, F, b, N, K), M, N, K, c)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(c.cpu().numpy().astype(np.float64), ka @ kb.T)
    ref, _ = orc.gemm_nt_reference(a, b, oc, M, N, K)
    np.testing.assert_array_equal(ref, ka @ kb.T)


@pytest.mark.parametrize("grid", [INT4, E1M2, E2M1])
def test_gemm_mx32_exact_on_representable_products(env, grid):
    # MX32 operands with random codes and E8M0 scales 2^-2 .. 2^2: every
    # product is a small integer times a power of two at least 2^-5 and every
    # partial sum stays below 2^19 in magnitude, so the fp32 result is exact;
    # covers the K positions and scales of every lane of the scaled MFMA
    torch, F, orc = env
    rng = np.random.default_rng(41 + grid)
    M, N, K = 96, 160, 384
    fc, oc = cfgs(F, orc, grid, RTNE, MX32, 0, 0, 0)
    top = 4 if grid == E2M1C else 7

    def layout(rows):
        k = rng.integers(-top, top + 1, size=(rows, K))
        nib = (np.where(k < 0, 8 | -k, k) if grid != INT4 else k & 15).astype(np.uint8)
        codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
        scales = rng.integers(125, 130, size=(rows, K // 32)).astype(np.uint8)
        q = (codes, scales, np.ones(1, np.float32))
        return q, orc.dequantize(*q, rows, K, oc).astype(np.float64)

    (a, xa), (b, xb) = layout(M), layout(N)
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    F.ufp4_gemm_nt(fc, upload(torch, F, a, M, K, MX32), upload(torch, F, b, N, K, MX32), M, N, K, c)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(c.cpu().numpy().astype(np.float64), xa @ xb.T)


def test_gemm_degenerate_shapes(env):
    torch, F, orc = env
    fc, oc = cfgs(F, orc)
    a = F.alloc_layout(16, 32, NV16)
    a.tensor_scale.fill_(1.0)
    c = torch.full((16, 16), 5.0, dtype=torch.float32, device="cuda")
    F.ufp4_gemm_nt(fc, a, a, 16, 16, 0, c)  # K = 0: zeros
    F.ufp4_gemm_nt(fc, a, a, 0, 16, 32, c)  # M = 0: nothing written
    torch.cuda.synchronize()
    assert bool((c == 0).all())


@pytest.mark.parametrize("recipe", [0, 1, 2])
def test_training_gemms_under_recipes(env, recipe):
    # each operand of fwd_y, bwd_dx and bwd_dw quantized on the GPU with the
    # configuration and layout its recipe preset gives (bit-exact against the
    # oracle with the same configuration), then multiplied by ufp4_gemm_nt
    # (within the fp32 accumulation bound of the float64 product of the
    # oracle's dequantized operands)
    torch, F, orc = env
    T, I, O = 256, 192, 160
    tens = {F.TENSOR_X: synth.activation(T, I, seed=11), F.TENSOR_W: synth.weight(O, I, seed=12),
            F.TENSOR_DY: synth.output_grad(T, O, seed=13)}
    for gemm in (F.GEMM_FWD_Y, F.GEMM_BWD_DX, F.GEMM_BWD_DW):
        say(f"[recipe] recipe={recipe} gemm={gemm}")
        qs, oqs, dims = [], [], []
        for operand in (F.OPERAND_A, F.OPERAND_B):
            fc, layout, tensor = F.ufp4_recipe_config(recipe, gemm, operand, rht_seed=5, sr_seed=9)
            oc = orc.config(fc.grid, fc.rounding, fc.scaling, fc.rht, fc.rht_seed, fc.sr_seed)
            xb = tens[tensor]
            row, col = gpu_rowcol(env, xb, fc)
            q = row if layout == ROW else col
            oq = orc.quantize(xb, oc, layout)
            np.testing.assert_array_equal(q.codes.cpu().numpy(), oq[0])
            np.testing.assert_array_equal(q.scales.cpu().numpy(), oq[1])
            assert q.tensor_scale.cpu().numpy()[0] == oq[2][0]
            R, C = xb.shape
            qs.append(q)
            oqs.append(oq)
            dims.append((R, C) if layout == ROW else (C, R))
        (M, K), (N, Kb) = dims
        assert K == Kb
        ref, mag = orc.gemm_nt_reference(oqs[0], oqs[1], oc, M, N, K)
        c = torch.empty((M, N), dtype=torch.float32, device="cuda")
        F.ufp4_gemm_nt(fc, qs[0], qs[1], M, N, K, c)
        torch.cuda.synchronize()
        err = np.abs(c.cpu().numpy().astype(np.float64) - ref)
        bound = (K + 4) * 2.0 ** -24 * mag + 1e-30
        assert (err <= bound).all(), f"max err/bound {float((err / bound).max()):.3g}"


# -------------------------------------------------------------- single pass
@pytest.mark.parametrize("stride", [2, 3, 7])
@pytest.mark.parametrize("rounding", [RTNE, SR])
def test_single_pass_left_tiles(env, schedule, stride, rounding):
    # tiles whose workgroup leaves them (forced from the host) are reloaded
    # and quantized by the workgroups that stay: bit for bit the same output
    torch, F, orc = env
    schedule(SINGLE_PASS, stride)
    R, C = 1040, 1024  # 4 bands x 9 row tiles, the last one ragged
    say(f"[single pass] {R}x{C} left stride={stride} rnd={rounding}")
    xb = synth.activation(R, C, seed=40 + stride)
    fc, oc = cfgs(F, orc, E1M2, rounding, NV16, 1, 5, 6)
    row, col = gpu_rowcol(env, xb, fc)
    assert_layout_equal(row, orc.quantize(xb, oc, ROW), f"row stride {stride}")
    assert_layout_equal(col, orc.quantize(xb, oc, COL), f"col stride {stride}")


def test_single_pass_more_tiles_than_the_device_holds(env, schedule):
    # 16384 x 2048 is 1024 tiles, twice what the device holds at once: the
    # first workgroups find tiles not started, leave theirs after the grace
    # period and exit; the later ones find every tile started and quantize
    # the left tiles too
    torch, F, orc = env
    schedule(SINGLE_PASS)
    R, C = 16384, 2048
    say(f"[single pass] {R}x{C} oversubscribed")
    xb = synth.activation(R, C, seed=44)
    fc, oc = cfgs(F, orc, E1M2, RTNE, NV16, 1, 2, 2)
    row, col = gpu_rowcol(env, xb, fc)
    assert_layout_equal(row, orc.quantize(xb, oc, ROW), "row")
    assert_layout_equal(col, orc.quantize(xb, oc, COL), "col")


def test_single_pass_workspace_reuse_across_shapes(env, schedule):
    # one workspace, calls on different shapes and layouts in turn: each
    # call's exchange words carry its own generation
    torch, F, orc = env
    schedule(SINGLE_PASS)
    ws = F.Workspace(1024, 1024)
    for R, C, seed in ((512, 512, 1), (256, 1024, 2), (1024, 768, 3), (512, 512, 4)):
        say(f"[single pass] reuse {R}x{C}")
        xb = synth.activation(R, C, seed=seed)
        fc, oc = cfgs(F, orc, E1M2, RTNE, NV16, 1, seed, seed)
        x = to_dev(torch, xb)
        row, col = F.alloc_layout(R, C, NV16), F.alloc_layout(C, R, NV16)
        F.ufp4_quantize_rowcol(x, fc, row, col, ws)
        rq = F.alloc_layout(R, C, NV16)
        F.ufp4_quantize(x, fc, rq, ws)
        torch.cuda.synchronize()
        assert_layout_equal(row, orc.quantize(xb, oc, ROW), f"row {R}x{C}")
        assert_layout_equal(col, orc.quantize(xb, oc, COL), f"col {R}x{C}")
        assert_layout_equal(rq, orc.quantize(xb, oc, ROW), f"row only {R}x{C}")
    assert ws.status() == 0


def test_workspace_status_words(env, schedule):
    # the status word is planted from the host (no fault is provoked): the
    # device writes 0, 6 (grouped offsets rejected) or 7 (a single-pass
    # exchange that did not complete); anything else is a corrupt workspace
    torch, F, orc = env
    ws = F.Workspace(256, 256)
    for word, want in ((0, 0), (6, 6), (7, 7), (5, 4), (0xDEAD, 4)):
        ws.buf[4:8] = torch.tensor([word], dtype=torch.int32).view(torch.uint8).cuda()
        assert ws.status() == want, (word, want)
    # a later single-pass call clears a stale failure and leaves a valid output
    schedule(SINGLE_PASS)
    ws.buf[4:8] = torch.tensor([7], dtype=torch.int32).view(torch.uint8).cuda()
    xb = synth.activation(256, 256, seed=3)
    fc, oc = cfgs(F, orc, E1M2, RTNE, NV16, 1, 3, 3)
    x = to_dev(torch, xb)
    row, col = F.alloc_layout(256, 256, NV16), F.alloc_layout(256, 256, NV16)
    F.ufp4_quantize_rowcol(x, fc, row, col, ws)
    assert ws.status() == 0
    assert_layout_equal(row, orc.quantize(xb, oc, ROW), "row")
    assert_layout_equal(col, orc.quantize(xb, oc, COL), "col")


# ------------------------------------------------------------------ grouped
def gpu_grouped(env, xb, offsets, fc, row=True, col=True):
    torch, F, _ = env
    R, C = xb.shape
    E = len(offsets) - 1
    B = 32 if fc.scaling == MX32 else 16
    coff = F.ufp4_grouped_col_offsets(offsets, B)
    Rp = int(coff[-1])
    x = to_dev(torch, xb)
    off = torch.from_numpy(np.asarray(offsets, np.int64)).cuda()
    rq = F.alloc_layout(R, C, fc.scaling, E) if row else None
    cq = F.alloc_layout(C, Rp, fc.scaling, E) if col else None
    ws = F.Workspace(R, C, E)
    F.ufp4_quantize_grouped(x, off, Rp, fc, rq, cq, ws)
    assert ws.status() == 0
    return rq, cq, coff


@pytest.mark.parametrize("scaling", [NV16, MX32])
@pytest.mark.parametrize("rounding", [RTNE, SR])
def test_grouped_small(env, scaling, rounding):
    torch, F, orc = env
    counts = np.array([0, 5, 16, 37, 1, 130, 0, 23, 64, 200, 3])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    xb = synth.activation(int(offsets[-1]), 320, seed=12)
    say(f"[grouped] E={len(counts)} rows={offsets[-1]} scl={scaling} rnd={rounding}")
    fc, oc = cfgs(F, orc, E1M2, rounding, scaling, 1, rht_seed=6, sr_seed=7)
    rq, cq, coff = gpu_grouped(env, xb, offsets, fc)
    (rc, rs, rts), (cc, cs, cts), ocoff = orc.quantize_grouped(xb, offsets, oc)
    np.testing.assert_array_equal(coff, ocoff)
    assert_layout_equal(rq, (rc, rs, rts), "grouped row")
    assert_layout_equal(cq, (cc, cs, cts), "grouped col")


def test_grouped_many_segments(env):
    # 1000 ragged segments (many empty or of one row), near the limit of 1024
    torch, F, orc = env
    rng = np.random.default_rng(14)
    counts = rng.integers(0, 6, size=1000) * rng.integers(0, 2, size=1000)
    counts[rng.integers(0, 1000, size=20)] = rng.integers(17, 300, size=20)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    xb = synth.activation(int(offsets[-1]), 256, seed=15)
    say(f"[grouped] E=1000 rows={offsets[-1]}")
    fc, oc = cfgs(F, orc, E1M2, SR, NV16, 1, rht_seed=8, sr_seed=8)
    rq, cq, coff = gpu_grouped(env, xb, offsets, fc)
    (rc, rs, rts), (cc, cs, cts), ocoff = orc.quantize_grouped(xb, offsets, oc)
    np.testing.assert_array_equal(coff, ocoff)
    assert_layout_equal(rq, (rc, rs, rts), "grouped row, 1000 segments")
    assert_layout_equal(cq, (cc, cs, cts), "grouped col, 1000 segments")


def test_grouped_single_outputs_and_bad_offsets(env):
    torch, F, orc = env
    counts = np.array([17, 0, 48])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    xb = synth.activation(int(offsets[-1]), 64, seed=13)
    fc, oc = cfgs(F, orc)
    (rc, rs, rts), (cc, cs, cts), _ = orc.quantize_grouped(xb, offsets, oc)
    rq, _, _ = gpu_grouped(env, xb, offsets, fc, row=True, col=False)
    assert_layout_equal(rq, (rc, rs, rts), "row only")
    _, cq, _ = gpu_grouped(env, xb, offsets, fc, row=False, col=True)
    assert_layout_equal(cq, (cc, cs, cts), "col only")
    # non-monotone offsets: the device detects it and writes nothing
    bad = np.array([0, 40, 20, 65], np.int64)
    R, C = xb.shape
    x = to_dev(torch, xb)
    rqb = F.alloc_layout(R, C, NV16, 3)
    rqb.codes.fill_(0xAB)
    ws = F.Workspace(R, C, 3)
    F.ufp4_quantize_grouped(x, torch.from_numpy(bad).cuda(), 96, fc, rqb, None, ws)
    assert ws.status() == 6
    assert bool((rqb.codes == 0xAB).all())


@pytest.mark.parametrize("grid", [E1M2, INT4, E2M1, E2M1C])
@pytest.mark.parametrize("rounding", [RTNE, SR])
@pytest.mark.parametrize("rht", [1, 0])
def test_grouped_delayed_matches_oracle(env, grid, rounding, rht):
    # per-segment provided maxima: the segment's own, larger, smaller
    # (saturating), zero and non-finite; codes, scales, tensor scales and the
    # per-segment maxima written for the next call against the oracle
    torch, F, orc = env
    counts = np.array([0, 5, 16, 37, 1, 130, 0, 23, 64, 200, 3])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    E = len(counts)
    xb = synth.activation(int(offsets[-1]), 320, seed=17)
    say(f"[grouped delayed] grid={grid} rnd={rounding} rht={rht}")
    fc, oc = cfgs(F, orc, grid, rounding, NV16, rht, rht_seed=6, sr_seed=7)
    *_, own = orc.quantize_grouped_given_amax(xb, offsets, oc, np.ones((E, 2), np.float32))
    rng = np.random.default_rng(grid * 4 + rounding * 2 + rht)
    given = (own * rng.choice([1.0, 3.0, 0.3], size=own.shape)).astype(np.float32)
    given[1, 0], given[2, 1], given[5, 0] = 0.0, np.inf, -1.0
    (rc, rs, rts), (cc, cs, cts), coff, seen = orc.quantize_grouped_given_amax(xb, offsets, oc, given)
    R, C = xb.shape
    Rp = int(coff[-1])
    x = to_dev(torch, xb)
    off = torch.from_numpy(offsets).cuda()
    rq, cq = F.alloc_layout(R, C, NV16, E), F.alloc_layout(C, Rp, NV16, E)
    a_in = torch.from_numpy(given.copy()).cuda()
    a_out = torch.full((E, 2), -1.0, dtype=torch.float32, device="cuda")
    ws = F.Workspace(R, C, E)
    F.ufp4_quantize_grouped_delayed(x, off, Rp, fc, a_in, a_out, rq, cq, ws)
    assert ws.status() == 0
    assert_layout_equal(rq, (rc, rs, rts), "grouped delayed row")
    assert_layout_equal(cq, (cc, cs, cts), "grouped delayed col")
    np.testing.assert_array_equal(a_out.cpu().numpy().view(np.uint32), seen.view(np.uint32))


def test_grouped_delayed_single_layouts_and_bad_offsets(env):
    torch, F, orc = env
    counts = np.array([17, 0, 48, 9])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    E = len(counts)
    xb = synth.activation(int(offsets[-1]), 64, seed=18)
    fc, oc = cfgs(F, orc, E1M2, RTNE, NV16, 1, 3, 3)
    *_, own = orc.quantize_grouped_given_amax(xb, offsets, oc, np.ones((E, 2), np.float32))
    (rc, rs, rts), (cc, cs, cts), coff, _ = orc.quantize_grouped_given_amax(xb, offsets, oc, own)
    R, C = xb.shape
    Rp = int(coff[-1])
    x = to_dev(torch, xb)
    off = torch.from_numpy(offsets).cuda()
    a_in = torch.from_numpy(own.copy()).cuda()
    a_out = torch.zeros((E, 2), dtype=torch.float32, device="cuda")
    ws = F.Workspace(R, C, E)
    rq = F.alloc_layout(R, C, NV16, E)
    F.ufp4_quantize_grouped_delayed(x, off, Rp, fc, a_in, a_out, rq, None, ws)
    assert_layout_equal(rq, (rc, rs, rts), "row only")
    got = a_out.cpu().numpy()
    assert np.array_equal(got[:, 0], own[:, 0]) and np.all(got[:, 1] == 0)  # column layout not requested
    cq = F.alloc_layout(C, Rp, NV16, E)
    F.ufp4_quantize_grouped_delayed(x, off, Rp, fc, a_in, None, None, cq, ws)
    assert_layout_equal(cq, (cc, cs, cts), "col only")
    bad = torch.from_numpy(np.array([0, 40, 20, 60, 74], np.int64)).cuda()
    rqb = F.alloc_layout(R, C, NV16, E)
    rqb.codes.fill_(0xAB)
    F.ufp4_quantize_grouped_delayed(x, bad, Rp, fc, a_in, None, rqb, None, ws)
    assert ws.status() == 6
    assert bool((rqb.codes == 0xAB).all())


def test_roof_hook_writes_every_output_byte(env):
    # the bandwidth reference writes zeros over every code and block-scale
    # byte of both layouts (which start as 0xAB) and leaves the tensor scales
    torch, F, orc = env
    R, C = 384, 768
    x = to_dev(torch, synth.activation(R, C, seed=19))
    row, col = F.alloc_layout(R, C, NV16), F.alloc_layout(C, R, NV16)
    for q in (row, col):
        q.codes.fill_(0xAB)
        q.scales.fill_(0xAB)
        q.tensor_scale.fill_(2.0)
    F.ufp4_roof_rowcol(x, row, col)
    torch.cuda.synchronize()
    for q in (row, col):
        assert int(q.codes.count_nonzero()) == 0 and int(q.scales.count_nonzero()) == 0
        assert bool((q.tensor_scale == 2.0).all())
    with pytest.raises(F.Ufp4Error):
        F.ufp4_roof_rowcol(x[:, :512].contiguous()[:200], row, col)


# ------------------------------------------------------- dequantize / stats
@pytest.mark.parametrize("grid", [E1M2, INT4, E2M1, E2M1C])
@pytest.mark.parametrize("scaling", [NV16, MX32])
def test_dequantize_bit_exact(env, grid, scaling):
    torch, F, orc = env
    R, C = 128, 256
    xb = synth.activation(R, C, seed=21)
    fc, oc = cfgs(F, orc, grid, RTNE, scaling, 1, rht_seed=2)
    row, col = gpu_rowcol(env, xb, fc)
    for q, rows, cols in ((row, R, C), (col, C, R)):
        for inv in (False, True):
            out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
            F.ufp4_dequantize(q, rows, cols, fc, inv, out)
            want = orc.dequantize(q.codes.cpu().numpy(), q.scales.cpu().numpy(),
                                  q.tensor_scale.cpu().numpy(), rows, cols, oc, inverse_rht=inv)
            np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))


def assert_stats_close(g, o, floor):
    for k in ("n", "n_saturated", "n_nonfinite", "n_zero_scale"):
        assert g[k] == o[k], k
    assert g["code_hist"] == o["code_hist"]
    assert g["amax"] == o["amax"]
    for k in ("sqnr_db", "mean_signed_err", "mean_signed_err_grid", "alpha"):
        a, b = g[k], o[k]
        assert abs(a - b) <= 1e-6 * max(abs(a), abs(b)) + floor, (k, a, b)


@pytest.mark.parametrize("grid", [E1M2, INT4, E2M1, E2M1C])
@pytest.mark.parametrize("layout", [ROW, COL])
def test_stats_match_oracle(env, grid, layout):
    torch, F, orc = env
    R, C = 256, 512
    xb = synth.weight(R, C, seed=2)
    fc, oc = cfgs(F, orc, grid, RTNE, NV16, 1, rht_seed=2)
    row, col = gpu_rowcol(env, xb, fc)
    q = row if layout == ROW else col
    g = F.ufp4_stats(to_dev(torch, xb), layout, fc, q, F.Workspace(R, C))
    o = orc.stats(xb, layout, oc, q.codes.cpu().numpy(), q.scales.cpu().numpy(), q.tensor_scale.cpu().numpy())
    floor = 1e-6 * float(np.mean(np.abs(synth.bf16_to_f32(xb))))
    assert_stats_close(g, o, floor)
