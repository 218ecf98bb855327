"""GPU parity at the five named workloads' full sizes, in the launch
configuration the benchmark times (one call through the C ABI).

The oracle finishes every workload in seconds to tens of seconds, so codes,
scales and tensor scales are compared in full, the MoE workload (268M
elements, 64 ragged segments) included: every segment, both layouts, every
per-segment tensor scale.
"""
import sys
import time

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

E1M2, INT4, E2M1, E2M1C = 0, 1, 2, 3
RTNE, SR = 0, 1
NV16, MX32 = 0, 1
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


def to_dev(torch, xb):
    return torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).cuda()


def eq(name, got, want):
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        raise AssertionError(f"{name}: {len(bad)} entries differ, first {bad[:5].tolist()}")


def check_layout(name, q, ref):
    c, s, t = ref
    eq(name + " codes", q.codes.cpu().numpy(), c)
    eq(name + " scales", q.scales.cpu().numpy(), s)
    eq(name + " tensor scale", q.tensor_scale.cpu().numpy()[: t.size].view(np.uint32), t.view(np.uint32))


def test_activation_rowcol_8192x2048(env):
    torch, F, orc = env
    say("[full] activation 8192x2048 RHT E1M2 RTNE row+col")
    xb = synth.activation(8192, 2048, seed=1)
    fc = F.config(E1M2, RTNE, NV16, 1, 1, 1)
    oc = orc.config(E1M2, RTNE, NV16, 1, 1, 1)
    x = to_dev(torch, xb)
    row, col = F.alloc_layout(8192, 2048, NV16), F.alloc_layout(2048, 8192, NV16)
    F.ufp4_quantize_rowcol(x, fc, row, col, F.Workspace(8192, 2048))
    torch.cuda.synchronize()
    t = time.time()
    ref_row, ref_col = orc.quantize(xb, oc, ROW), orc.quantize(xb, oc, COL)
    check_layout("row", row, ref_row)
    check_layout("col", col, ref_col)
    say(f"  oracle+compare {time.time() - t:.1f}s")
    # delayed scaling, chained as in training: a first call under a stale
    # maximum, then a call under the first one's tile maxima = the exact path
    say("[full] activation 8192x2048 delayed, chained")
    n = F.ufp4_amax_tiles(8192, 2048)
    a1 = torch.full((n, 2), -1.0, dtype=torch.float32, device="cuda")
    a2 = torch.full((n, 2), -1.0, dtype=torch.float32, device="cuda")
    stale = torch.tensor([[3.0, 5.0]], dtype=torch.float32, device="cuda")
    F.ufp4_quantize_delayed(x, fc, stale, a1, row, col)
    F.ufp4_quantize_delayed(x, fc, a1, a2, row, col)
    torch.cuda.synchronize()
    check_layout("delayed row", row, ref_row)
    check_layout("delayed col", col, ref_col)
    assert torch.equal(a1, a2) and bool((a1 >= 0).all())


@pytest.mark.parametrize("grid,rounding,scaling", [(E2M1, RTNE, NV16), (E2M1, SR, NV16), (E2M1, RTNE, MX32),
                                                    (E2M1, SR, MX32), (INT4, RTNE, NV16), (E1M2, RTNE, MX32)])
def test_activation_variants_rowcol_8192x2048(env, grid, rounding, scaling):
    # the grid, rounding and scaling variants of the headline call, as the
    # benchmark's variant legs launch them (one row+column call)
    torch, F, orc = env
    say(f"[full] activation 8192x2048 RHT grid={grid} rnd={rounding} scl={scaling} row+col")
    xb = synth.activation(8192, 2048, seed=1)
    fc = F.config(grid, rounding, scaling, 1, 1, 1)
    oc = orc.config(grid, rounding, scaling, 1, 1, 1)
    x = to_dev(torch, xb)
    row, col = F.alloc_layout(8192, 2048, scaling), F.alloc_layout(2048, 8192, scaling)
    F.ufp4_quantize_rowcol(x, fc, row, col, F.Workspace(8192, 2048))
    torch.cuda.synchronize()
    check_layout("row", row, orc.quantize(xb, oc, ROW))
    check_layout("col", col, orc.quantize(xb, oc, COL))


def test_weight_grid_sweep_2048x8192(env):
    torch, F, orc = env
    xb = synth.weight(2048, 8192, seed=2)
    x = to_dev(torch, xb)
    ws = F.Workspace(2048, 8192)
    floor = 1e-6 * float(np.mean(np.abs(synth.bf16_to_f32(xb))))
    for grid in (E1M2, INT4, E2M1, E2M1C):
        for rht in (1, 0):
            say(f"[full] weight 2048x8192 grid={grid} rht={rht} row + stats")
            fc = F.config(grid, RTNE, NV16, rht, 2, 2)
            oc = orc.config(grid, RTNE, NV16, rht, 2, 2)
            row = F.alloc_layout(2048, 8192, NV16)
            F.ufp4_quantize(x, fc, row, ws)
            ref = orc.quantize(xb, oc, ROW)
            check_layout("row", row, ref)
            g = F.ufp4_stats(x, ROW, fc, row, ws)
            o = orc.stats(xb, ROW, oc, *ref)
            for k in ("n", "n_saturated", "n_nonfinite", "n_zero_scale", "code_hist", "amax"):
                assert g[k] == o[k], k
            for k in ("sqnr_db", "mean_signed_err", "mean_signed_err_grid", "alpha"):
                assert abs(g[k] - o[k]) <= 1e-6 * max(abs(g[k]), abs(o[k])) + floor, (k, g[k], o[k])
            say(f"  sqnr={g['sqnr_db']:.3f} dB alpha={g['alpha']:.6f} mse_grid={g['mean_signed_err_grid']:.5f}")


def test_output_grad_sr_rowcol_16384x4096(env):
    torch, F, orc = env
    say("[full] output gradient 16384x4096 RHT E1M2 SR row+col")
    xb = synth.output_grad(16384, 4096, seed=3)
    fc = F.config(E1M2, SR, NV16, 1, 3, 3)
    oc = orc.config(E1M2, SR, NV16, 1, 3, 3)
    x = to_dev(torch, xb)
    row, col = F.alloc_layout(16384, 4096, NV16), F.alloc_layout(4096, 16384, NV16)
    F.ufp4_quantize_rowcol(x, fc, row, col, F.Workspace(16384, 4096))
    torch.cuda.synchronize()
    t = time.time()
    check_layout("row", row, orc.quantize(xb, oc, ROW))
    check_layout("col", col, orc.quantize(xb, oc, COL))
    say(f"  oracle+compare {time.time() - t:.1f}s")


def test_moe_grouped_65536x4096(env):
    torch, F, orc = env
    say("[full] MoE 65536x4096, 64 experts, RHT E1M2 RTNE grouped row+col")
    xb, offsets = synth.moe_activation(8192, 4096, 64, 8, seed=4)
    counts = np.diff(offsets)
    E = counts.size
    coff = F.ufp4_grouped_col_offsets(offsets, 16)
    Rp = int(coff[-1])
    fc = F.config(E1M2, RTNE, NV16, 1, 4, 4)
    oc = orc.config(E1M2, RTNE, NV16, 1, 4, 4)
    x = to_dev(torch, xb)
    rq = F.alloc_layout(xb.shape[0], 4096, NV16, E)
    cq = F.alloc_layout(4096, Rp, NV16, E)
    ws = F.Workspace(xb.shape[0], 4096, E)
    F.ufp4_quantize_grouped(x, torch.from_numpy(offsets).cuda(), Rp, fc, rq, cq, ws)
    assert ws.status() == 0
    torch.cuda.synchronize()
    t = time.time()
    (rc, rs, rts), (cc, cs, cts), ocoff = orc.quantize_grouped(xb, offsets, oc)
    np.testing.assert_array_equal(coff, ocoff)
    say(f"  oracle {time.time() - t:.1f}s; comparing all {E} segments, both layouts")
    eq("row codes", rq.codes.cpu().numpy(), rc)
    eq("row scales", rq.scales.cpu().numpy(), rs)
    eq("row tensor scales", rq.tensor_scale.cpu().numpy()[:E].view(np.uint32), rts.view(np.uint32))
    eq("col codes", cq.codes.cpu().numpy(), cc)
    eq("col scales", cq.scales.cpu().numpy(), cs)
    eq("col tensor scales", cq.tensor_scale.cpu().numpy()[:E].view(np.uint32), cts.view(np.uint32))

    # grouped delayed scaling, chained as in training: a first call under
    # stale per-segment maxima, then a call under the first one's maxima,
    # which are the segments' own: the exact grouped path, bit for bit
    say("[full] MoE 65536x4096 grouped delayed, chained")
    stale = torch.full((E, 2), 3.0, dtype=torch.float32, device="cuda")
    a1 = torch.full((E, 2), -1.0, dtype=torch.float32, device="cuda")
    a2 = torch.full((E, 2), -1.0, dtype=torch.float32, device="cuda")
    offd = torch.from_numpy(offsets).cuda()
    F.ufp4_quantize_grouped_delayed(x, offd, Rp, fc, stale, a1, rq, cq, ws)
    F.ufp4_quantize_grouped_delayed(x, offd, Rp, fc, a1, a2, rq, cq, ws)
    torch.cuda.synchronize()
    assert ws.status() == 0
    assert torch.equal(a1, a2) and bool((a1 >= 0).all())
    eq("delayed row codes", rq.codes.cpu().numpy(), rc)
    eq("delayed row scales", rq.scales.cpu().numpy(), rs)
    eq("delayed row tensor scales", rq.tensor_scale.cpu().numpy()[:E].view(np.uint32), rts.view(np.uint32))
    eq("delayed col codes", cq.codes.cpu().numpy(), cc)
    eq("delayed col scales", cq.scales.cpu().numpy(), cs)
    eq("delayed col tensor scales", cq.tensor_scale.cpu().numpy()[:E].view(np.uint32), cts.view(np.uint32))
