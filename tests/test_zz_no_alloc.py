"""The no-allocation entry point (ufp4_quantize_rowcol_noalloc) against the
workspace entry point it varies (ufp4_quantize_rowcol), through the C ABI:
bit-identical codes, scales and tensor scales on calls in a row, each later
call on a smaller tensor than the one before (the shared scratch array keeps
the earlier call's contents), under each schedule; the call captured in a
HIP graph and replayed; and the size limit, rejected before anything is
enqueued."""
import ctypes
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

E1M2, INT4, E2M1 = 0, 1, 2
RTNE, SR = 0, 1
NV16, MX32 = 0, 1
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


def same(torch, a, b, what):
    assert torch.equal(a.codes, b.codes), f"{what}: codes"
    assert torch.equal(a.scales, b.scales), f"{what}: scales"
    assert torch.equal(a.tensor_scale.view(torch.int32), b.tensor_scale.view(torch.int32)), f"{what}: tensor scale"


@pytest.mark.parametrize("sched", [AUTO, TWO_PASS, SINGLE_PASS])
def test_noalloc_matches_workspace_call(env, sched):
    torch, F, orc = env
    F.ufp4_set_schedule(sched, 0)
    try:
        # larger first, then smaller: the second call finds the first one's
        # partials and exchange words in the scratch array
        for R, C, seed, grid, rnd, scl in ((2048, 2048, 1, E1M2, RTNE, NV16), (512, 768, 2, E1M2, SR, NV16),
                                           (256, 256, 3, E2M1, RTNE, NV16), (128, 512, 4, INT4, RTNE, MX32)):
            say(f"[noalloc] sched={sched} {R}x{C} grid={grid} rnd={rnd} scl={scl}")
            xb = synth.activation(R, C, seed=seed)
            x = torch.from_numpy(xb.view(np.int16)).cuda()
            fc = F.config(grid, rnd, scl, 1, seed, seed)
            ra, ca = F.alloc_layout(R, C, scl), F.alloc_layout(C, R, scl)
            rb, cb = F.alloc_layout(R, C, scl), F.alloc_layout(C, R, scl)
            rb.codes.fill_(0x5A)
            cb.codes.fill_(0x5A)
            F.ufp4_quantize_rowcol(x, fc, ra, ca, F.Workspace(R, C))
            F.ufp4_quantize_rowcol_noalloc(x, fc, rb, cb)
            torch.cuda.synchronize()
            same(torch, ra, rb, "row")
            same(torch, ca, cb, "col")
        # the last call's output against the oracle as well
        oc = orc.config(INT4, RTNE, MX32, 1, 4, 4)
        c, s, t = orc.quantize(xb, oc, 0)
        assert np.array_equal(rb.codes.cpu().numpy(), c) and np.array_equal(rb.scales.cpu().numpy(), s)
    finally:
        F.ufp4_set_schedule(AUTO, 0)


@pytest.mark.parametrize("sched", [AUTO, TWO_PASS])
def test_noalloc_in_a_captured_graph(env, sched):
    # the callers this entry point is for capture it in a HIP graph: the
    # call is captured once and replayed three times, with eager calls on
    # another tensor in between (which leave their own contents in the
    # scratch array); every replay matches the workspace call's output
    torch, F, _ = env
    F.ufp4_set_schedule(sched, 0)
    try:
        R, C = 1024, 1536
        xb = synth.output_grad(R, C, seed=7)
        x = torch.from_numpy(xb.view(np.int16)).cuda()
        fc = F.config(E1M2, SR, NV16, 1, 7, 7)
        ra, ca = F.alloc_layout(R, C, NV16), F.alloc_layout(C, R, NV16)
        F.ufp4_quantize_rowcol(x, fc, ra, ca, F.Workspace(R, C))
        rb, cb = F.alloc_layout(R, C, NV16), F.alloc_layout(C, R, NV16)
        other = torch.from_numpy(synth.activation(512, 512, seed=8).view(np.int16)).cuda()
        ro, co = F.alloc_layout(512, 512, NV16), F.alloc_layout(512, 512, NV16)
        F.ufp4_quantize_rowcol_noalloc(x, fc, rb, cb)  # first use on the device happens eagerly
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            F.ufp4_quantize_rowcol_noalloc(x, fc, rb, cb)
        torch.cuda.synchronize()
        for rep in range(3):
            say(f"[noalloc graph] sched={sched} replay {rep}")
            rb.codes.fill_(0x5A)
            cb.codes.fill_(0x5A)
            F.ufp4_quantize_rowcol_noalloc(other, fc, ro, co)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            same(torch, ra, rb, f"row, replay {rep}")
            same(torch, ca, cb, f"col, replay {rep}")
    finally:
        F.ufp4_set_schedule(AUTO, 0)


def test_noalloc_size_limit(env):
    torch, F, _ = env
    # 2^24 x 16384 needs far more than the 1 MiB scratch array: rejected on
    # the host (the pointers are never used)
    fc = F.config(E1M2, RTNE, NV16, 1, 0, 0)
    q = F.ufp4_qtensor(16, 16, 16)
    rc = F.lib.ufp4_quantize_rowcol_noalloc(16, 1 << 24, 16384, 16384, ctypes.byref(fc), q, q, None)
    assert rc == 4
