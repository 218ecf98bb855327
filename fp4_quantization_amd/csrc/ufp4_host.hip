// ufp4_host.hip -- host-side helpers of the quantization launches: the
// folded random signs of the transform and the launch geometry.  Host code
// only (no kernels), so a sanitized host build of the C ABI can link it
// without the device code.
//
// The signs: d_j = -1 iff bit j of word 0 of Philox4x32-10(key = rht_seed,
// counter = (0, 0, 2, 0)) is set; one vector per seed, shared by every block
// ("Shrinkage Bias: The Hidden Geometric Trap in FP4 Training" (zhichai.net),
// "Key points": random Hadamard transform; Philox4x32-10 from Salmon et al.,
// SC'11).
#include "ufp4_internal.hpp"

namespace ufp4 {

uint32_t rht_sign_mask(uint64_t seed) {
  // word 0 of Philox4x32-10(key = seed, counter = (0, 0, 2, 0))
  uint32_t c0 = 0, c1 = 0, c2 = 2, c3 = 0;
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  for (int r = 0; r < 10; ++r) {
    const uint64_t a = (uint64_t)0xD2511F53u * c0, b = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(b >> 32) ^ c1 ^ k0, n1 = (uint32_t)b;
    const uint32_t n2 = (uint32_t)(a >> 32) ^ c3 ^ k1, n3 = (uint32_t)a;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c0 & 0xFFFFu;
}

void fill_rht_signs(uint64_t seed, QuantParams& p) {
  const uint32_t mask = rht_sign_mask(seed);
  float d[16];
  for (int j = 0; j < 16; ++j) d[j] = ((mask >> j) & 1u) ? -1.0f : 1.0f;
  RhtSigns& S = p.sg;
  for (int q = 0; q < 8; ++q) S.q1[q] = d[2 * q] * d[2 * q + 1];
  for (int g = 0; g < 4; ++g) S.q2[g] = d[4 * g] * d[4 * g + 2];
  for (int g = 0; g < 2; ++g) S.q3[g] = d[8 * g] * d[8 * g + 4];
  S.q4 = d[0] * d[8];
  S.fin = 0.25f * d[0];
  for (int h = 0; h < 2; ++h) {
    for (int q = 0; q < 4; ++q) p.hs[h].q1[q] = S.q1[4 * h + q];
    for (int g = 0; g < 2; ++g) p.hs[h].q2[g] = S.q2[2 * h + g];
    p.hs[h].q3 = S.q3[h];
  }
  // stage 4 across a lane pair: the even lane (positions 0..7) computes
  // a + q4 b; the odd lane computes b - q4 a = -q4 (a - q4 b).
  p.s4[0] = S.q4;
  p.s4[1] = -S.q4;
  p.fin_lane[0] = S.fin;
  p.fin_lane[1] = S.fin * -S.q4;
}

int64_t grid_size_quant(int64_t rows, int64_t cols, int32_t groups, int32_t block, int32_t* n_band,
                        int32_t* n_tiles) {
  const int64_t nb = (cols + kBandCols - 1) / kBandCols;
  int64_t nt;
  if (groups <= 1) {
    const int64_t P = (rows + block - 1) / block * block;
    nt = (P + kTileRows - 1) / kTileRows;
  } else {
    // sum over segments of ceil(roundup(M_e, B) / 128) <= ceil((rows + B*E)/128) + E
    nt = (rows + (int64_t)block * groups + kTileRows - 1) / kTileRows + groups;
  }
  if (nt < 1) nt = 1;
  *n_band = (int32_t)nb;
  *n_tiles = (int32_t)nt;
  const int64_t work = nb * nt;
  return (work + kNumXcd - 1) / kNumXcd * kNumXcd;
}

}  // namespace ufp4
