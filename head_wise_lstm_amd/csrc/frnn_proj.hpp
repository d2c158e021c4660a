// Input projection of the multi-layer LSTM ("5.3 LSTM": x_t . Wi + bias_ih + bias_hh) for all T
// steps at once, as one MFMA GEMM:  C[M][Nc] (fp32) = A[M][K] . Bw[K][Nc] + b1[Nc] + b2[Nc].
// A is bf16 or fp32 (converted to bf16 while staged), Bw and the biases bf16, row-major.
//
// 128 x 128 output tile per workgroup, K staged 32 at a time through LDS, 4 waves in a 2 x 2
// arrangement each owning 64 x 64 (4 x 4 tiles of v_mfma_f32_16x16x32_bf16). A is staged row-major
// (the A fragment is 8 consecutive k of one row), Bw transposed to [n][k] (the B fragment is 8
// consecutive k of one column), so every fragment read is one 16-byte LDS access.
#pragma once

#include "frnn_device.hpp"

namespace frnn {

struct ProjArgs {
  int M, Nc, K;
  const void* A;
  int a_f32;
  long long lda;
  const uint16_t* Bw;
  long long ldb;
  const uint16_t* b1;
  const uint16_t* b2;
  float* C;
  long long ldc;
};

constexpr int PJ_BM = 128, PJ_BN = 128, PJ_BK = 32, PJ_LS = PJ_BK + 8;

__global__ void __launch_bounds__(256) proj_gemm_kernel(ProjArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[PJ_BM * PJ_LS];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[PJ_BN * PJ_LS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, quad = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const long long m0 = (long long)blockIdx.y * PJ_BM;
  const int n0 = blockIdx.x * PJ_BN;

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < p.K; k0 += PJ_BK) {
    // A tile: 128 rows x 32 k; thread -> row tid/2, 16 consecutive k.
    {
      const int r = tid >> 1, kh = (tid & 1) * 16;
      const long long gm = m0 + r;
      uint16_t v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int gk = k0 + kh + i;
        float f = 0.0f;
        if (gm < p.M && gk < p.K) {
          const long long off = gm * p.lda + gk;
          f = p.a_f32 ? reinterpret_cast<const float*>(p.A)[off] : bf2f(reinterpret_cast<const uint16_t*>(p.A)[off]);
        }
        v[i] = p.a_f32 ? f2bf(f) : (uint16_t)(__float_as_uint(f) >> 16);
      }
#pragma unroll
      for (int i = 0; i < 16; i += 2)
        *reinterpret_cast<uint32_t*>(&As[r * PJ_LS + kh + i]) = (uint32_t)v[i] | ((uint32_t)v[i + 1] << 16);
    }
    // Bw tile: 32 k x 128 n, stored transposed; thread -> k row tid/8, 16 consecutive n.
    {
      const int kr = tid >> 3, nb = (tid & 7) * 16;
      const int gk = k0 + kr;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int gn = n0 + nb + i;
        const uint16_t v = (gk < p.K && gn < p.Nc) ? p.Bw[(long long)gk * p.ldb + gn] : (uint16_t)0;
        Bs[(nb + i) * PJ_LS + kr] = v;
      }
    }
    __syncthreads();
    bf16x8_t af[4], bfr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = *reinterpret_cast<const bf16x8_t*>(&As[(wm * 64 + i * 16 + col) * PJ_LS + 8 * quad]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[(wn * 64 + j * 16 + col) * PJ_LS + 8 * quad]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(af[i], bfr[j], acc[i][j]);
    __syncthreads();
  }
  // Epilogue: lane holds rows 4*quad + r of column col of every 16 x 16 tile.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int gn = n0 + wn * 64 + j * 16 + col;
    if (gn >= p.Nc) continue;
    const float bias = (p.b1 ? bf2f(p.b1[gn]) : 0.0f) + (p.b2 ? bf2f(p.b2[gn]) : 0.0f);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const long long gm = m0 + wm * 64 + i * 16 + 4 * quad + r;
        if (gm < p.M) p.C[gm * p.ldc + gn] = acc[i][j][r] + bias;
      }
    }
  }
}

}  // namespace frnn
