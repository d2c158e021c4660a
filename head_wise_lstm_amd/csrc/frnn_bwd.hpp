// Backward (back-propagation through time) of the head-wise recurrence, for gfx950.
//
// Given the forward's inputs, its fp32 states output and the gradients dstates / dlast of its
// two outputs, this computes dWx, dR, db and dstates0 (the chain rule of the forward cell
// equations; the pages print no gradient formulas). The work splits into
//   1. h_{t-1} . R for every step at once: every h_{t-1} is already in the forward's states, so
//      the pre-activations are recomputed by one MFMA GEMM per head (M = T*B rows (t, b), K = D,
//      N = G*D), not by a serial loop;
//   2. the serial part, t = T-1 .. 0: a pointwise kernel turns the step's incoming gradient into
//      dWx and da (the gradient of the step's h.R part), then an MFMA kernel forms the gradient
//      that reaches h_{t-1}, dh = sum_g da_g . R_g^T;
//   3. dR = sum over (t, b) of h_{t-1}^T da, one GEMM per head over K = T*B, with db from a row of
//      ones appended to h^T.
// Operands of the contractions are bf16 (fp32 for fp32 inputs) with fp32 accumulation, like the
// forward; every carried gradient and every output is fp32.
#pragma once

#include "frnn_device.hpp"

namespace frnn {

struct BwdArgs {
  int B, T, N, D, cell;
  int f32;        // operands fp32 (else bf16)
  int Kp;         // T*B rounded up to a multiple of 32: rows of the (t, b) operand buffers
  const void* Wx;
  long long wx_sb, wx_st;
  const void* R;
  long long r_sg, r_sn, r_sd;
  const void* bias;
  const void* s0_h;
  const void* s0_c;
  long long s0_sb;
  const float* st_h;  // forward states [B,T,N,D] (h), and c for the LSTM
  const float* st_c;
  long long st_sb, st_st;
  const float* ds_h;  // gradient of states (or null)
  const float* ds_c;
  const float* dl_h;  // gradient of last_states (or null)
  const float* dl_c;
  long long last_sb;
  float* dWx;         // [B,T,G,N,D] (or null)
  float* ds0_h;       // [B,N,D] slices of dstates0 (or null)
  float* ds0_c;
  void* hprev;        // [N][Kp][D] operand: row t*B + b = h_{t-1} of batch row b
  const float* hr;    // [N][T*B][G*D]: h_{t-1} . R recomputed
  void* da;           // [N][Kp][G*D] operand: gradient of the h.R part of step t
  float* dhrec;       // [B][N][D]: gradient reaching h through R from the step after
  float* carry;       // [B][N][D]: LSTM dc, GRU direct dh carried to the step before
};

__device__ __forceinline__ void st_op(void* p, long long i, float v, bool f32) {
  if (f32) reinterpret_cast<float*>(p)[i] = v;
  else reinterpret_cast<uint16_t*>(p)[i] = f2bf(v);
}

// hprev[n][t*B + b][d] = h_{t-1}[b][n][d] (the initial state for t = 0), in the operand type;
// rows T*B .. Kp-1 are zero.
__global__ void __launch_bounds__(256) bwd_hprev_kernel(BwdArgs a) {
  const long long total = (long long)a.N * a.Kp * a.D;
  const bool f32 = a.f32;
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (long long)gridDim.x * 256) {
    const int d = (int)(idx % a.D);
    const long long r = idx / a.D;
    const int row = (int)(r % a.Kp);
    const int n = (int)(r / a.Kp);
    float v = 0.0f;
    if (row < a.T * a.B) {
      const int t = row / a.B, b = row % a.B;
      if (t > 0) v = a.st_h[(long long)b * a.st_sb + (long long)(t - 1) * a.st_st + (long long)n * a.D + d];
      else if (a.s0_h) v = ld_f(a.s0_h, (long long)b * a.s0_sb + (long long)n * a.D + d, f32);
    }
    st_op(a.hprev, idx, v, f32);
  }
}

// Step t of the serial part: one thread per (b, n, unit), consecutive threads on consecutive
// units. Reads the recomputed h.R, Wx, bias and the forward states of the step, adds the
// incoming gradients, and writes dWx, da (operand type, for the dh kernel and dR) and the carry.
__global__ void __launch_bounds__(256) bwd_gate_kernel(BwdArgs a, int t) {
  const long long total = (long long)a.B * a.N * a.D;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int u = (int)(idx % a.D);
  const long long r = idx / a.D;
  const int n = (int)(r % a.N);
  const int b = (int)(r / a.N);
  const int N = a.N, D = a.D, G = cell_gates(a.cell);
  const bool f32 = a.f32;
  const long long tb = (long long)t * a.B + b;
  const float* hr = a.hr + ((long long)n * a.T * a.B + tb) * G * D + u;
  const long long wbase = (long long)b * a.wx_sb + (long long)t * a.wx_st + (long long)n * D + u;
  const long long sidx = (long long)b * a.st_sb + (long long)t * a.st_st + (long long)n * D + u;
  const long long lidx = (long long)b * a.last_sb + (long long)n * D + u;
  float pre[4] = {0.f, 0.f, 0.f, 0.f}, wx[4] = {0.f, 0.f, 0.f, 0.f}, bb[4] = {0.f, 0.f, 0.f, 0.f};
  for (int g = 0; g < G; ++g) {
    pre[g] = hr[(long long)g * D];
    wx[g] = ld_f(a.Wx, wbase + (long long)g * N * D, f32);
    bb[g] = a.bias ? ld_f(a.bias, (long long)(g * N + n) * D + u, f32) : 0.0f;
  }
  float dh = a.dhrec[idx];
  if (a.ds_h) dh += a.ds_h[sidx];
  if (t == a.T - 1 && a.dl_h) dh += a.dl_h[lidx];
  float dw[4] = {0.f, 0.f, 0.f, 0.f}, dav[4];
  if (a.cell == CELL_LSTM) {
    const float ig = sigmoid_f(pre[0] + wx[0] + bb[0]);
    const float fg = sigmoid_f(pre[1] + wx[1] + bb[1]);
    const float zg = tanh_f(pre[2] + wx[2] + bb[2]);
    const float og = sigmoid_f(pre[3] + wx[3] + bb[3]);
    const float ct = a.st_c[sidx];
    const float cp = t > 0 ? a.st_c[sidx - a.st_st]
                           : (a.s0_c ? ld_f(a.s0_c, (long long)b * a.s0_sb + (long long)n * D + u, f32) : 0.0f);
    float dc = a.carry[idx];
    if (a.ds_c) dc += a.ds_c[sidx];
    if (t == a.T - 1 && a.dl_c) dc += a.dl_c[lidx];
    const float tc = tanh_f(ct);
    const float dct = dc + dh * og * (1.0f - tc * tc);
    dw[0] = dct * zg * ig * (1.0f - ig);
    dw[1] = dct * cp * fg * (1.0f - fg);
    dw[2] = dct * ig * (1.0f - zg * zg);
    dw[3] = dh * tc * og * (1.0f - og);
    a.carry[idx] = dct * fg;
    for (int g = 0; g < 4; ++g) dav[g] = dw[g];
  } else if (a.cell == CELL_GRU) {
    dh += a.carry[idx];
    const float rg = sigmoid_f(pre[0] + wx[0] + bb[0]);
    const float zg = sigmoid_f(pre[1] + wx[1] + bb[1]);
    const float q = pre[2] + bb[2];
    const float ng = tanh_f(wx[2] + rg * q);
    const float hp = t > 0 ? a.st_h[sidx - a.st_st]
                           : (a.s0_h ? ld_f(a.s0_h, (long long)b * a.s0_sb + (long long)n * D + u, f32) : 0.0f);
    const float dq = dh * (1.0f - zg) * (1.0f - ng * ng);
    dw[0] = dq * q * rg * (1.0f - rg);
    dw[1] = dh * (hp - ng) * zg * (1.0f - zg);
    dw[2] = dq;
    dav[0] = dw[0];
    dav[1] = dw[1];
    dav[2] = dq * rg;
    a.carry[idx] = dh * zg;
  } else {
    const float ht = a.st_h[sidx];
    dw[0] = dh * (1.0f - ht * ht);
    dav[0] = dw[0];
  }
  if (a.dWx)
    for (int g = 0; g < G; ++g) a.dWx[wbase + (long long)g * N * D] = dw[g];
  const long long drow = ((long long)n * a.Kp + tb) * G * D + u;
  for (int g = 0; g < G; ++g) st_op(a.da, drow + (long long)g * D, dav[g], f32);
}

// dh of step t-1: dhrec[b][n][d] = sum_g sum_e da[n][t*B + b][g*D + e] * R[g][n][d][e].
// MFMA with A = R rows (16 values of d; k = (g, e), 32 at a time within one gate: 16 contiguous
// bytes of a row of R per lane) and B = da^T (batch in the 16 columns). Grid (D/16, ceil(B/16),
// N); the 4 waves take k-tiles 4 apart and meet in LDS.
template <bool F32>
__global__ void __launch_bounds__(256) bwd_dh_kernel(BwdArgs a, int t) {
  __shared__ f32x4_t part[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, quad = lane >> 4;
  const int G = cell_gates(a.cell), D = a.D;
  const int d0 = blockIdx.x * 16, b0 = blockIdx.y * 16, n = blockIdx.z;
  const int KW = F32 ? 4 : 32;
  const int KT = G * D / KW;
  const bool colv = b0 + col < a.B;
  const long long drow = ((long long)n * a.Kp + (long long)t * a.B + b0 + col) * G * D;
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int kt = wave; kt < KT; kt += 8) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = kt + 4 * h;
      if (k >= KT) break;
      const int g = (k * KW) / D, e0 = (k * KW) % D;
      const long long rrow = (long long)g * a.r_sg + (long long)n * a.r_sn + (long long)(d0 + col) * a.r_sd + e0;
      if constexpr (F32) {
        const float av = reinterpret_cast<const float*>(a.R)[rrow + quad];
        const float bv = colv ? reinterpret_cast<const float*>(a.da)[drow + k * KW + quad] : 0.0f;
        if (h == 0) acc0 = mfma_f32(av, bv, acc0);
        else acc1 = mfma_f32(av, bv, acc1);
      } else {
        const u32x4_t av = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(a.R) + rrow + 8 * quad);
        u32x4_t bv = {0u, 0u, 0u, 0u};
        if (colv) bv = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(a.da) + drow + k * KW + 8 * quad);
        if (h == 0) acc0 = mfma_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv), acc0);
        else acc1 = mfma_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv), acc1);
      }
    }
  }
  part[wave][lane] = acc0 + acc1;
  __syncthreads();
  if (wave != 0 || !colv) return;
  const f32x4_t s = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
  *reinterpret_cast<f32x4_t*>(a.dhrec + ((long long)(b0 + col) * a.N + n) * D + d0 + 4 * quad) = s;
}

// dstates0 from what reaches the initial state: h through R (plus the GRU's direct part), and
// the LSTM's carried dc.
__global__ void __launch_bounds__(256) bwd_final_kernel(BwdArgs a) {
  const long long total = (long long)a.B * a.N * a.D;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  if (a.ds0_h) a.ds0_h[idx] = a.dhrec[idx] + (a.cell == CELL_GRU ? a.carry[idx] : 0.0f);
  if (a.ds0_c && a.cell == CELL_LSTM) a.ds0_c[idx] = a.carry[idx];
}

// dR[g][n][d][e] = tmp[n][d][g*D + e] and db[g][n][e] = tmp[n][D][g*D + e] (tmp: [N][D+1][G*D]
// fp32, the dR GEMM's output with its row of ones).
__global__ void __launch_bounds__(256) bwd_scatter_kernel(const float* tmp, int N, int D, int G, float* dR, float* db) {
  const long long total = (long long)N * (D + 1) * G * D;
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (long long)gridDim.x * 256) {
    const int col = (int)(idx % (G * D));
    const long long r = idx / (G * D);
    const int d = (int)(r % (D + 1));
    const int n = (int)(r / (D + 1));
    const int g = col / D, e = col % D;
    if (d < D) {
      if (dR) dR[(((long long)g * N + n) * D + d) * D + e] = tmp[idx];
    } else if (db) {
      db[((long long)g * N + n) * D + e] = tmp[idx];
    }
  }
}

// Row d = D of h^T: ones (db as one more row of the dR GEMM).
__global__ void __launch_bounds__(256) bwd_ones_row_kernel(void* hT, int N, int D, int Kp, int f32) {
  const long long total = (long long)N * Kp;
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (long long)gridDim.x * 256) {
    const int k = (int)(idx % Kp);
    const int n = (int)(idx / Kp);
    st_op(hT, ((long long)n * (D + 1) + D) * Kp + k, 1.0f, f32);
  }
}

// Plain fp32 GEMM for the fp32 inputs: C[M][Nc] = A[M][K] . Bt[Nc][K]^T, one 16 x 16 tile per
// wave on v_mfma_f32_16x16x4f32, operands read straight from memory (K a multiple of 4).
__global__ void __launch_bounds__(256) gemm_f32_kernel(int M, int Nc, int K, const float* A, long long lda,
                                                       const float* Bt, long long ldb, float* C, long long ldc) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, quad = lane >> 4;
  const int tn = (Nc + 15) / 16;
  const long long tile = (long long)blockIdx.x * 4 + wave;
  if (tile >= (long long)((M + 15) / 16) * tn) return;
  const int m0 = (int)(tile / tn) * 16, n0 = (int)(tile % tn) * 16;
  const bool mv = m0 + col < M, nv = n0 + col < Nc;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < K; k += 4) {
    const float av = mv ? A[(long long)(m0 + col) * lda + k + quad] : 0.0f;
    const float bv = nv ? Bt[(long long)(n0 + col) * ldb + k + quad] : 0.0f;
    acc = mfma_f32(av, bv, acc);
  }
  if (!nv) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 4 * quad + i;
    if (m < M) C[(long long)m * ldc + n0 + col] = acc[i];
  }
}

}  // namespace frnn
