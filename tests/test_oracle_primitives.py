"""Pins of the CPU oracle's primitives against things other than itself.

Each test pins one primitive to a library routine, a brute-force search, a
closed form or a value the pages print (tests/golden/).  None re-uses the
oracle's own code path for the expected value.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_grids():
    grids = {}
    with open(os.path.join(GOLDEN, "grids.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, *vals = line.split()
            grids[name] = np.array([float(v) for v in vals])
    return grids


# ------------------------------------------------------------------ Philox
ROCRAND_SRC = r"""
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
int main() {
  unsigned long long key, sub, off;
  while (scanf("%llx %llx %llx", &key, &sub, &off) == 3) {
    rocrand_device::philox4x32_10_engine eng(key, sub, off);
    unsigned a = eng.next(), b = eng.next(), c = eng.next(), d = eng.next();
    printf("%08x %08x %08x %08x\n", a, b, c, d);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def rocrand_philox(tmp_path_factory):
    """rocRAND's Philox4x32-10 engine (library header), built for the host."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("rocRAND header / hipcc not available")
    d = tmp_path_factory.mktemp("rocrand")
    src = d / "rr.cpp"
    src.write_text(ROCRAND_SRC)
    exe = d / "rr"
    subprocess.run([hipcc, "--offload-arch=gfx950", str(src), "-o", str(exe)], check=True,
                   capture_output=True)

    def run(queries):
        inp = "".join(f"{k:x} {s:x} {o:x}\n" for k, s, o in queries)
        out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True).stdout
        return [[int(w, 16) for w in line.split()] for line in out.strip().splitlines()]

    return run


def test_philox_block_matches_rocrand(orc, rocrand_philox):
    # rocRAND engine(seed, subsequence, offset): key = seed, counter =
    # (offset/4 as 64 bits, subsequence as 64 bits), words in order.
    rng = np.random.default_rng(123)
    cases = [(0, 0, 0, 0, 0, 0), (0xFFFFFFFF,) * 6]
    for _ in range(40):
        cases.append(tuple(int(v) for v in rng.integers(0, 2**32, size=6, dtype=np.uint64)))
    queries = [((k1 << 32) | k0, (c3 << 32) | c2, ((c1 << 32) | c0) * 4)
               for c0, c1, c2, c3, k0, k1 in cases]
    # offset*4 overflows 64 bits when c1 >= 2^30; rocRAND counts modulo 2^64 too
    queries = [(k, s, o & (2**64 - 1)) for k, s, o in queries]
    ref = rocrand_philox(queries)
    for (c0, c1, c2, c3, k0, k1), (k, s, o), want in zip(cases, queries, ref):
        ctr = [(o // 4) & 0xFFFFFFFF, (o // 4) >> 32, c2, c3]
        got = orc.philox4x32_10(ctr, [k0, k1])
        assert list(got) == want, (cases, got, want)


def test_sr_word_and_signs_match_rocrand(orc, rocrand_philox):
    # SR word of element i in stream s == rocRAND engine(seed, subsequence=s, offset=i).next()
    queries, expect = [], []
    for seed in (0, 3, 0xDEADBEEFCAFEF00D):
        for stream in (0, 1):
            for i in (0, 1, 2, 3, 4, 5, 1023, 2**32 + 7, 2**40 + 2):
                queries.append((seed, stream, i))
                expect.append(orc.sr_word(seed, i, stream))
    ref = rocrand_philox(queries)
    assert [r[0] for r in ref] == expect
    # RHT signs: bit j of word 0 of counter (0,0,2,0)
    for seed in (0, 1, 2, 3, 4, 12345):
        w0 = rocrand_philox([(seed, 2, 0)])[0][0]
        want = np.array([-1 if (w0 >> j) & 1 else 1 for j in range(16)], np.int8)
        np.testing.assert_array_equal(orc.rht_signs(seed), want)


def test_philox_words_uniform(orc):
    # chi-square uniformity of 2^16 words over 256 bins of the top byte
    words = np.array([orc.sr_word(7, i, 0) for i in range(1 << 16)], dtype=np.uint64)
    hist = np.bincount((words >> 24).astype(np.int64), minlength=256)
    e = (1 << 16) / 256
    chi2 = float(((hist - e) ** 2 / e).sum())
    assert chi2 < 400.0  # df=255: p ~ 1e-7 at 400


# -------------------------------------------------------------------- FWHT
def sylvester16():
    i = np.arange(16)
    pc = np.array([[bin(a & b).count("1") for b in i] for a in i])
    return np.where(pc % 2 == 0, 1, -1)


def test_fwht_is_sylvester_hadamard(orc):
    H = np.stack([orc.fwht16_stages(np.eye(16, dtype=np.float32)[j]) for j in range(16)], axis=1)
    np.testing.assert_array_equal(H, sylvester16())
    np.testing.assert_array_equal(H @ H.T, 16 * np.eye(16))


def test_rht_integer_inputs_exact(orc):
    # small integer inputs: every butterfly is exact, so the result equals
    # (1/4) H D x computed in exact integer arithmetic
    rng = np.random.default_rng(5)
    H = sylvester16()
    for seed in range(6):
        s = orc.rht_signs(seed)
        x = rng.integers(-1000, 1000, size=16)
        v = orc.rht16(x.astype(np.float32), s)
        np.testing.assert_array_equal(v.astype(np.float64), (H @ (s * x)) / 4.0)


def test_rht_one_hot_closed_form(orc):
    H = sylvester16()
    s = orc.rht_signs(9)
    for j in range(16):
        for c in (1.0, -3.0, 2.0 ** -100, 1e30):
            x = np.zeros(16, np.float32)
            x[j] = c
            v = orc.rht16(x, s)
            np.testing.assert_array_equal(v, np.float32(c / 4.0) * s[j] * H[:, j])


def test_rht_inverse_roundtrip_and_parseval(orc):
    rng = np.random.default_rng(11)
    for seed in range(4):
        s = orc.rht_signs(seed)
        for _ in range(200):
            x = rng.standard_normal(16).astype(np.float32)
            v = orc.rht16(x, s)
            xr = orc.inverse_rht16(v, s)
            n = np.linalg.norm(x.astype(np.float64))
            assert np.max(np.abs(xr.astype(np.float64) - x)) <= 1e-6 * n
            assert abs(np.sum(v.astype(np.float64) ** 2) - n * n) <= 1e-6 * n * n


def test_rht_rounding_within_bound(orc):
    # random bf16 inputs: each output within 4 roundings of the exact value
    rng = np.random.default_rng(12)
    H = sylvester16()
    s = orc.rht_signs(1)
    for _ in range(300):
        x = synth.bf16_to_f32(synth.f32_to_bf16(rng.standard_normal(16).astype(np.float32) *
                                                 np.float32(10.0) ** rng.integers(-3, 4, 16)))
        v = orc.rht16(x, s).astype(np.float64)
        exact = (H @ (s * x.astype(np.float64))) / 4.0
        bound = 4 * 2.0 ** -24 * (np.abs(x).sum() / 4.0)
        assert np.all(np.abs(v - exact) <= bound + 1e-45)


def test_rht_outputs_are_multiples_of_the_bf16_quantum(orc):
    # Every input is a multiple of 2^-133 (the smallest bf16 step), so every
    # fp32 sum and difference of the butterfly is one too (rounding never
    # goes below the operands' common step), and the transform's outputs,
    # after the final 1/4, are multiples of 2^-135.  The quantizer's
    # single-product scaling relies on this: the 1/4 is exact and a nonzero
    # value never falls below 2^-135.  Inputs mix bf16 subnormals with values
    # up to 2^100, random signs.
    rng = np.random.default_rng(13)
    s = orc.rht_signs(3)
    for _ in range(400):
        mag = rng.integers(0, 0x7180, 16)  # bf16 magnitude patterns: 0, subnormals .. 2^100
        mag[rng.random(16) < 0.3] = rng.integers(1, 0x80, 1)[0]  # some subnormals in most blocks
        x = synth.bf16_to_f32((mag | (rng.integers(0, 2, 16) << 15)).astype(np.uint16))
        q = orc.rht16(x, s).astype(np.float64) * 2.0 ** 135
        assert np.all(np.isfinite(q)) and np.all(q == np.round(q))


# -------------------------------------------------------------------- E4M3
def _e4m3_values():
    vals = []
    for c in range(127):
        e, m = c >> 3, c & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def test_e4m3_decode_matches_torch(orc):
    torch = pytest.importorskip("torch")
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    got = np.array([orc.e4m3_decode(c) for c in range(256)], np.float32)
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_e4m3_encode_roundtrip_all_codes(orc):
    for c in range(127):
        assert orc.e4m3_encode(orc.e4m3_decode(c)) == c


def test_e4m3_encode_vs_torch_and_brute_force(orc):
    torch = pytest.importorskip("torch")
    vals = _e4m3_values()
    # every fp32 within +-64 ulps of every E4M3 value and every midpoint, plus a
    # strided sweep of all non-negative fp32 below 464
    pts = np.concatenate([vals, (vals[:-1] + vals[1:]) / 2, [464.0]]).astype(np.float32)
    bits = pts.view(np.uint32).astype(np.int64)
    near = (bits[:, None] + np.arange(-64, 65)[None, :]).reshape(-1)
    sweep = np.arange(0, 0x43E80001, 997, dtype=np.int64)
    allbits = np.unique(np.concatenate([near, sweep]))
    allbits = allbits[(allbits >= 0) & (allbits <= 0x43E80000)]
    q = allbits.astype(np.uint32).view(np.float32)
    got = orc.e4m3_encode_n(q)
    ref = torch.from_numpy(q.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, ref)
    # brute force nearest, ties to even code, on the targeted points
    qn = q[: near.size // 4].astype(np.float64)
    d = np.abs(qn[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = np.where(d == best, np.arange(127)[None, :], 1 << 20)
    even = np.where((cand & 1) == 0, cand, 1 << 20).min(axis=1)
    want = np.where(even < (1 << 20), even, cand.min(axis=1))
    np.testing.assert_array_equal(got[: qn.size], want)


def test_e4m3_saturates(orc):
    for q in (448.0, 460.0, 464.0, 470.0, 1e10, float("inf")):
        assert orc.e4m3_encode(q) == 0x7E
    assert orc.e4m3_encode(0.0) == 0 and orc.e4m3_encode(-1.0) == 0


# ------------------------------------------------------------ grid rounding
GRID_IDS = {"E1M2": 0, "INT4": 1, "E2M1": 2, "E2M1_CLAMP": 3}
ALL_GRIDS = ["E1M2", "INT4", "E2M1", "E2M1_CLAMP"]


def _grid_mags(orc):
    g = _golden_grids()
    e2m1 = g["E2M1"]
    # The clamped grid is E2M1 limited to its uniformly spaced part: the
    # printed E2M1 magnitudes up to the first step that is not 0.5.
    steps = np.diff(e2m1)
    uniform_end = int(np.argmax(steps != 0.5)) + 1
    return {"E1M2": g["E1M2"], "E2M1": e2m1, "INT4": np.arange(8.0), "E2M1_CLAMP": e2m1[:uniform_end]}


def _brute_force_codes(y, mags, int4):
    """Nearest magnitude by exhaustive search; tie -> even index; |y| >= Qmax -> Qmax;
    NaN -> code 0; magnitude 0 -> code 0."""
    a = np.abs(y.astype(np.float64))
    with np.errstate(invalid="ignore"):
        d = np.abs(a[:, None] - mags[None, :])
    best = d.min(axis=1, keepdims=True)
    idx = np.arange(len(mags))[None, :]
    ties = d == best
    even = np.where(ties & (idx % 2 == 0), idx, 99).min(axis=1)
    any_ = np.where(ties, idx, 99).min(axis=1)
    k = np.where(even < 99, even, any_)
    k = np.where(a >= mags[-1], len(mags) - 1, k)
    neg = np.signbit(y)
    if int4:
        code = np.where(neg, (16 - k) % 16, k)
    else:
        code = np.where(neg, 8 | k, k)
    code = np.where(k == 0, 0, code)
    code = np.where(np.isnan(y), 0, code)
    return code.astype(np.uint8)


@pytest.mark.parametrize("grid", ALL_GRIDS)
def test_rtne_exhaustive_bf16_vs_brute_force(orc, grid):
    y = synth.all_bf16_patterns()
    got = orc.round_f32(y, GRID_IDS[grid], 0)
    want = _brute_force_codes(y, _grid_mags(orc)[grid], grid == "INT4")
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("grid", ALL_GRIDS)
def test_code_values_match_printed_grid(orc, grid):
    mags = _grid_mags(orc)[grid]
    for k in range(len(mags)):
        assert orc.code_value(k, GRID_IDS[grid]) == mags[k]
        neg = (16 - k) % 16 if grid == "INT4" else 8 | k
        if k:
            assert orc.code_value(neg, GRID_IDS[grid]) == -mags[k]
    assert orc.grid_qmax(GRID_IDS[grid]) == mags[-1]


def _bucket_bias_fixture():
    with open(os.path.join(GOLDEN, "bucket_bias.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            fmt, q, left, right, mean = line.split()
            return fmt, float(q), float(left), float(right), float(mean)


def test_e2m1_bucket_bias_matches_page(orc):
    fmt, q, left, right, mean = _bucket_bias_fixture()
    assert fmt == "E2M1" and mean == (left - right) / 2
    n = 1 << 20
    y = (q - left + (np.arange(n) + 0.5) * (left + right) / n).astype(np.float32)
    codes = orc.round_f32(y, GRID_IDS["E2M1"], 0)
    vals = np.array([orc.code_value(c, 2) for c in range(16)])[codes]
    assert np.all(vals == q)
    assert abs(np.mean(vals - y.astype(np.float64)) - mean) < 1e-4


def test_clamped_e2m1_is_uniform_and_saturates_at_two(orc):
    mags = _grid_mags(orc)["E2M1_CLAMP"]
    assert np.array_equal(mags, [0.0, 0.5, 1.0, 1.5, 2.0]) and orc.grid_qmax(3) == 2.0
    # interior buckets are symmetric, as for E1M2: no rounding bias
    n = 1 << 20
    for q in (0.5, 1.0, 1.5):
        y = (q - 0.25 + (np.arange(n) + 0.5) * 0.5 / n).astype(np.float32)
        vals = np.array([orc.code_value(c, 3) for c in range(16)])[orc.round_f32(y, 3, 0)]
        assert np.all(vals == q) and abs(np.mean(vals - y.astype(np.float64))) < 1e-6
    # everything from 2 up to E2M1's own range ends at the largest code
    y = np.array([2.0, 2.4, 3.0, 5.9, 6.0, 1e30], np.float32)
    assert np.all(orc.round_f32(y, 3, 0) == 4) and np.all(orc.round_f32(-y, 3, 0) == 12)


def test_e1m2_bucket_unbiased(orc):
    # the uniform grid's q = 2.0 bucket is symmetric: [1.75, 2.25)
    n = 1 << 20
    y = (1.75 + (np.arange(n) + 0.5) * 0.5 / n).astype(np.float32)
    codes = orc.round_f32(y, GRID_IDS["E1M2"], 0)
    vals = np.array([orc.code_value(c, 0) for c in range(16)])[codes]
    assert np.all(vals == 2.0)
    assert abs(np.mean(vals - y.astype(np.float64))) < 1e-4


@pytest.mark.parametrize("grid", ["E1M2", "INT4", "E2M1"])
def test_stochastic_rounding_unbiased(orc, grid):
    gid = GRID_IDS[grid]
    mags = _grid_mags(orc)[grid]
    n = 10 ** 6
    table = np.array([orc.code_value(c, gid) for c in range(16)])
    ys = [mags[1] * 0.3, mags[2] + (mags[3] - mags[2]) * 1e-3, mags[3] + (mags[4] - mags[3]) * 0.999,
          -(mags[5] + (mags[6] - mags[5]) * 0.5), (mags[6] + mags[7]) / 2 + 0.01 * (mags[7] - mags[6])]
    for y0 in ys:
        y0 = float(np.float32(y0))
        codes = orc.round_f32(np.full(n, y0, np.float32), gid, 1, sr_seed=99)
        vals = table[codes]
        a = abs(y0)
        i = int(np.searchsorted(mags, a, side="right") - 1)
        lo, hi = mags[i], mags[i + 1]
        assert set(np.unique(np.abs(vals))) <= {lo, hi}
        p = (a - lo) / (hi - lo)
        sigma = (hi - lo) * np.sqrt(p * (1 - p) / n)
        assert abs(np.mean(vals) - y0) <= 3 * sigma + 1e-12, (y0, np.mean(vals), sigma)


def test_stochastic_rounding_exact_values_never_move(orc):
    for gid, mags in ((0, np.arange(8) * 0.5), (2, _golden_grids()["E2M1"])):
        y = np.repeat(mags.astype(np.float32), 1000)
        codes = orc.round_f32(y, gid, 1, sr_seed=3)
        vals = np.array([orc.code_value(c, gid) for c in range(16)])[codes]
        np.testing.assert_array_equal(vals, y)


def test_attenuation_fixture():
    # sanity of the compounding figure printed on the pages (used in docs only)
    with open(os.path.join(GOLDEN, "attenuation.txt")) as f:
        line = [ln for ln in f if not ln.startswith("#")][0].split()
    g, n, rem, tol = float(line[1]), int(line[3]), float(line[5]), float(line[7])
    assert abs(g ** n - rem) < tol
