"""GPU: the chain of quantized GEMMs that measures the compounding of the GEMM
gain ("Shrinkage Bias: The Hidden Geometric Trap in FP4 Training"
(zhichai.net), "Key points", compounding decay), and the fp32 -> bf16
conversion between its layers, against the oracle's chain."""
import sys

import numpy as np
import pytest

import synth
from test_oracle_tensor import _grid_input_and_block_permutations

pytestmark = pytest.mark.gpu

E1M2, INT4, E2M1 = 0, 1, 2
RTNE, NV16 = 0, 0


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp4_quantization_amd as F
    import fp4_quantization_amd.shrinkage as S
    import oracle
    oracle.lib()
    return torch, F, S, oracle


def dev(torch, hb):
    return torch.from_numpy(np.ascontiguousarray(hb).view(np.int16)).cuda()


def expected_bf16(f):
    # round to nearest, ties to even, on the bit pattern; NaN -> quiet NaN
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r[nan] = ((u[nan] >> 16) | 0x40) & 0xFFFF
    return r.astype(np.uint16)


def test_f32_to_bf16_bit_exact(env):
    torch, F, _, _ = env
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, size=1_000_003, dtype=np.uint64).astype(np.uint32)
    special = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFF800001, 0x7F800001,
                        0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F808001, 0x7F7FFFFF, 0x00008000, 0x00018000,
                        0x807FFFFF], np.uint32)
    bits[:special.size] = special
    f = bits.view(np.float32)
    for off in (0, 1):  # 16-byte aligned (vector path) and not
        say(f"[bf16] offset {off}")
        x = torch.from_numpy(f.copy()).cuda()[off:]
        got = F.ufp4_f32_to_bf16(x.contiguous() if off == 0 else x).cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(got, expected_bf16(f[off:].copy()))


@pytest.mark.parametrize("grid", [E1M2, INT4])
def test_chain_exact_case(env, grid):
    torch, F, S, orc = env
    T, D, L = 64, 64, 4
    k, h, Ws, perms = _grid_input_and_block_permutations(T, D, L, seed=5)
    r = S.shrinkage_chain(dev(torch, h), [dev(torch, w) for w in Ws], F.config(grid, RTNE, NV16, 0, 0, 0))
    o = orc.shrinkage_chain(h, Ws, orc.config(grid, RTNE, NV16, 0, 0, 0))
    np.testing.assert_array_equal(r["last_input"].cpu().numpy().view(np.uint16), o["last_input"])
    assert r["gain"] == [1.0] * L and r["alpha_a"] == [1.0] * L
    assert all(abs(e - 1.0) <= 2.0 ** -23 for e in r["eta"]), r["eta"]


@pytest.mark.parametrize("grid", [E1M2, E2M1])
@pytest.mark.parametrize("rht", [0, 1])
def test_chain_matches_oracle(env, grid, rht):
    # Layer 1 sees the same input on both sides: alpha to the statistics'
    # tolerance, eta to the fp32 accumulation of the GEMM.  Later layers see
    # inputs that may differ in rare bf16 roundings of the two GEMM results,
    # so gains agree to 2e-3.
    torch, F, S, orc = env
    T, D, L = 512, 256, 8
    say(f"[chain] grid={grid} rht={rht}")
    h0 = synth.activation(T, D, seed=21)
    Ws = [synth.orthogonal(D, seed=100 + i) for i in range(L)]
    r = S.shrinkage_chain(dev(torch, h0), [dev(torch, w) for w in Ws], F.config(grid, RTNE, NV16, rht, 3, 0))
    o = orc.shrinkage_chain(h0, Ws, orc.config(grid, RTNE, NV16, rht, 3, 0))
    for key in ("alpha_a", "alpha_b"):
        assert abs(r[key][0] - o[key][0]) <= 1e-6 * abs(o[key][0]), key
    assert abs(r["eta"][0] - o["eta"][0]) <= 1e-5
    for key in ("eta", "gain", "alpha_a", "alpha_b"):
        d = np.abs(np.array(r[key]) - np.array(o[key]))
        assert d.max() <= 2e-3, (key, d)
    # alpha of the weights does not depend on the chain
    np.testing.assert_allclose(r["alpha_b"], o["alpha_b"], rtol=1e-6)
