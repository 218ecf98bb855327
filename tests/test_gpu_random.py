"""Seeded random configurations through the C ABI against the oracle: shapes
(ragged tails, padded leading dimensions), grids, roundings, scalings, the
transform on or off, schedules, single and both layouts, and grouped calls
with random segment sizes.  Codes, scales and tensor scales bit for bit."""
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

AUTO, TWO_PASS, SINGLE_PASS = 0, 1, 2
ROW, COL = 0, 1


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


def check(q, ref, what):
    c, s, t = ref
    assert np.array_equal(q.codes.cpu().numpy(), c), f"{what}: codes"
    assert np.array_equal(q.scales.cpu().numpy(), s), f"{what}: scales"
    assert q.tensor_scale.cpu().numpy().view(np.uint32)[: t.size].tolist() == t.view(np.uint32).tolist(), \
        f"{what}: tensor scale"


def draw_input(rng, R, C):
    kind = rng.integers(0, 3)
    seed = int(rng.integers(0, 1 << 30))
    if kind == 0:
        return synth.activation(R, C, seed=seed)
    if kind == 1:
        return synth.weight(R, C, seed=seed)
    return synth.output_grad(R, C, seed=seed)


@pytest.mark.parametrize("case", range(24))
def test_random_dense(env, case):
    torch, F, orc = env
    rng = np.random.default_rng(1000 + case)
    scaling = int(rng.integers(0, 2))
    B = 32 if scaling == 1 else 16
    R = int(rng.integers(1, 80)) * B
    C = int(rng.integers(1, 60)) * B
    pad = int(rng.integers(0, 3)) * 8
    grid, rounding, rht = int(rng.integers(0, 4)), int(rng.integers(0, 2)), int(rng.integers(0, 2))
    rs, ss = int(rng.integers(0, 1 << 40)), int(rng.integers(0, 1 << 40))
    sched = int(rng.choice([AUTO, TWO_PASS, SINGLE_PASS]))
    both = bool(rng.integers(0, 4))  # mostly row+col
    say(f"[random {case}] {R}x{C} ld+{pad} grid={grid} rnd={rounding} scl={scaling} rht={rht} sched={sched} both={both}")
    xb = draw_input(rng, R, C)
    fc = F.config(grid, rounding, scaling, rht, rs, ss)
    oc = orc.config(grid, rounding, scaling, rht, rs, ss)
    buf = np.zeros((R, C + pad), np.uint16)
    buf[:, :C] = xb
    x = torch.from_numpy(buf.view(np.int16)).cuda()[:, :C]
    F.ufp4_set_schedule(sched, 0)
    try:
        ws = F.Workspace(R, C)
        row = F.alloc_layout(R, C, scaling)
        if both:
            col = F.alloc_layout(C, R, scaling)
            F.ufp4_quantize_rowcol(x, fc, row, col, ws)
        else:
            F.ufp4_quantize(x, fc, row, ws)
        torch.cuda.synchronize()
    finally:
        F.ufp4_set_schedule(AUTO, 0)
    check(row, orc.quantize(xb, oc, ROW), "row")
    if both:
        check(col, orc.quantize(xb, oc, COL), "col")


@pytest.mark.parametrize("case", range(8))
def test_random_grouped(env, case):
    torch, F, orc = env
    rng = np.random.default_rng(2000 + case)
    scaling = int(rng.integers(0, 2))
    B = 32 if scaling == 1 else 16
    E = int(rng.integers(1, 40))
    counts = rng.integers(0, 200, size=E) * (rng.random(E) > 0.2)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    C = int(rng.integers(1, 24)) * B
    grid, rounding, rht = int(rng.integers(0, 4)), int(rng.integers(0, 2)), int(rng.integers(0, 2))
    rs, ss = int(rng.integers(0, 1 << 40)), int(rng.integers(0, 1 << 40))
    say(f"[random grouped {case}] E={E} rows={offsets[-1]} C={C} grid={grid} rnd={rounding} scl={scaling} rht={rht}")
    xb = draw_input(rng, int(offsets[-1]), C)
    fc = F.config(grid, rounding, scaling, rht, rs, ss)
    oc = orc.config(grid, rounding, scaling, rht, rs, ss)
    coff = F.ufp4_grouped_col_offsets(offsets, B)
    Rp = int(coff[-1])
    R = xb.shape[0]
    x = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).cuda()
    rq, cq = F.alloc_layout(R, C, scaling, E), F.alloc_layout(C, Rp, scaling, E)
    ws = F.Workspace(R, C, E)
    F.ufp4_quantize_grouped(x, torch.from_numpy(offsets).cuda(), Rp, fc, rq, cq, ws)
    torch.cuda.synchronize()
    assert ws.status() == 0
    (rc, rsc, rts), (cc, csc, cts), ocoff = orc.quantize_grouped(xb, offsets, oc)
    np.testing.assert_array_equal(coff, ocoff)
    check(rq, (rc, rsc, rts), "grouped row")
    check(cq, (cc, csc, cts), "grouped col")
