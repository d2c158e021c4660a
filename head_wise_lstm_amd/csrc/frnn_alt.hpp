// Alternating forward recurrence for gfx950: per step, one MFMA kernel computes h.R for all heads
// and batch rows, then one coalesced pointwise kernel applies the gates. R is packed once per call
// into MFMA-fragment order, so every per-step operand load is a contiguous 1 KiB per wave.
//
// Tiles follow the fused design: a 16-row tile of R^T holds the four gate rows of four units
// (LSTM; GRU with a zero fourth row) or sixteen units (Elman); lane l of the MFMA result holds
// rows 4*(l/16)+i of batch column l%16.
#pragma once

#include "frnn_device.hpp"

namespace frnn {

struct AltArgs {
  int B, T, N, D, cell;
  int r_is_f32;  // R, bias and the exchanged h are fp32 (fp32 MFMA) or bf16 (bf16 MFMA)
  const void* Wx;
  int wx_f32;
  long long wx_sb, wx_st;
  const void* R;
  long long r_sg, r_sn, r_sd;
  const void* bias;
  const void* s0_h;
  const void* s0_c;
  int s0_f32;
  long long s0_sb, s0_sn;  // element strides of the initial states for b and n
  float* out_h;
  float* out_c;
  long long out_sb, out_st;
  float* last_h;
  float* last_c;
  long long last_sb, last_sn;
  int rev_n0;  // heads n >= rev_n0 run backwards in time: step t reads Wx and writes states at T-1-t
  void* rpack;    // packed R fragments: [N][TPH][KT][64][8 bf16] or [N][TPH][KT][64] fp32
  float* rh;      // h.R per step: LSTM, GRU [B][N][D][4]; Elman [B][N][D]
  void* hcur;     // current h, MFMA operand type: [N][B][D]
  float* ccur;    // current c (LSTM) or h in fp32 (GRU): [B][N][D]
};

// Initial state into the working buffers: hcur[n][b][d] (operand type), ccur[b][n][d] (the
// LSTM's c, the GRU's h).
__global__ void __launch_bounds__(256) alt_init_kernel(AltArgs a) {
  const long long total = (long long)a.B * a.N * a.D;
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (long long)gridDim.x * 256) {
    const int d = (int)(idx % a.D);
    const long long r = idx / a.D;
    const int n = (int)(r % a.N);
    const int b = (int)(r / a.N);
    const long long s = (long long)b * a.s0_sb + (long long)n * a.s0_sn + d;
    const float h = a.s0_h ? ld_f(a.s0_h, s, a.s0_f32) : 0.0f;
    const float c = a.cell == CELL_GRU ? h : a.s0_c ? ld_f(a.s0_c, s, a.s0_f32) : 0.0f;
    const long long hi = ((long long)n * a.B + b) * a.D + d;
    if (a.r_is_f32) reinterpret_cast<float*>(a.hcur)[hi] = h;
    else reinterpret_cast<uint16_t*>(a.hcur)[hi] = f2bf(h);
    a.ccur[idx] = c;
  }
}

// Per step: grid (TPH, ceil(B/16), N), one R^T tile per workgroup. The 4 waves take the tile's
// k-tiles 4 apart (wave w: w, w+4, ...), each with two accumulators, so that every wave has a
// quarter of the fragment loads in flight at once; the four partial sums meet in LDS.
template <bool F32>
__global__ void __launch_bounds__(256) alt_gemm_kernel(AltArgs a) {
  __shared__ f32x4_t part[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, quad = lane >> 4;
  const int GS = cell_slots(a.cell);
  const int TPH = GS * a.D / 16;
  const int tt = blockIdx.x;
  const int b0 = blockIdx.y * 16;
  const int n = blockIdx.z;
  const int KW = F32 ? 4 : 32;
  const int KT = a.D / KW;
  const bool colv = b0 + col < a.B;
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  if constexpr (F32) {
    const float* rp = reinterpret_cast<const float*>(a.rpack) + ((long long)n * TPH + tt) * KT * 64 + lane;
    const float* hp = reinterpret_cast<const float*>(a.hcur) + ((long long)n * a.B + b0 + col) * a.D + quad;
    int kt = wave;
    for (; kt + 4 < KT; kt += 8) {
      const float a0 = rp[(long long)kt * 64], a1 = rp[(long long)(kt + 4) * 64];
      const float h0 = colv ? hp[kt * 4] : 0.0f, h1 = colv ? hp[(kt + 4) * 4] : 0.0f;
      acc0 = mfma_f32(a0, h0, acc0);
      acc1 = mfma_f32(a1, h1, acc1);
    }
    if (kt < KT) acc0 = mfma_f32(rp[(long long)kt * 64], colv ? hp[kt * 4] : 0.0f, acc0);
  } else {
    const u32x4_t* rp = reinterpret_cast<const u32x4_t*>(a.rpack) + ((long long)n * TPH + tt) * KT * 64 + lane;
    const uint16_t* hp = reinterpret_cast<const uint16_t*>(a.hcur) + ((long long)n * a.B + b0 + col) * a.D + 8 * quad;
    int kt = wave;
    for (; kt + 4 < KT; kt += 8) {
      const u32x4_t a0 = rp[(long long)kt * 64], a1 = rp[(long long)(kt + 4) * 64];
      u32x4_t h0 = {0u, 0u, 0u, 0u}, h1 = {0u, 0u, 0u, 0u};
      if (colv) {
        h0 = *reinterpret_cast<const u32x4_t*>(hp + kt * 32);
        h1 = *reinterpret_cast<const u32x4_t*>(hp + (kt + 4) * 32);
      }
      acc0 = mfma_bf16(__builtin_bit_cast(bf16x8_t, a0), __builtin_bit_cast(bf16x8_t, h0), acc0);
      acc1 = mfma_bf16(__builtin_bit_cast(bf16x8_t, a1), __builtin_bit_cast(bf16x8_t, h1), acc1);
    }
    if (kt < KT) {
      u32x4_t h0 = {0u, 0u, 0u, 0u};
      if (colv) h0 = *reinterpret_cast<const u32x4_t*>(hp + kt * 32);
      acc0 = mfma_bf16(__builtin_bit_cast(bf16x8_t, rp[(long long)kt * 64]), __builtin_bit_cast(bf16x8_t, h0), acc0);
    }
  }
  part[wave][lane] = acc0 + acc1;
  __syncthreads();
  if (wave != 0 || !colv) return;
  const f32x4_t s = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
  const long long b = b0 + col;
  if (GS == 4) {
    const int u = 4 * tt + quad;
    *reinterpret_cast<f32x4_t*>(a.rh + ((b * a.N + n) * a.D + u) * 4) = s;
  } else {
    const int u = 16 * tt + 4 * quad;
    *reinterpret_cast<f32x4_t*>(a.rh + (b * a.N + n) * a.D + u) = s;
  }
}

// Per step: one thread per (b, n, unit); consecutive threads take consecutive units, so the Wx,
// bias, state and output accesses of a wave are contiguous.
__global__ void __launch_bounds__(256) alt_gate_kernel(AltArgs a, int t) {
  const long long total = (long long)a.B * a.N * a.D;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int u = (int)(idx % a.D);
  const long long r = idx / a.D;
  const int n = (int)(r % a.N);
  const long long b = r / a.N;
  const int N = a.N, D = a.D;
  const int tt = n >= a.rev_n0 ? a.T - 1 - t : t;  // the head's time direction
  const long long wbase = b * a.wx_sb + (long long)tt * a.wx_st;
  const long long o = b * a.out_sb + (long long)tt * a.out_st + (long long)n * D + u;
  const bool rf = a.r_is_f32;
  float h, c = 0.0f;
  if (a.cell == CELL_LSTM) {
    const f32x4_t rh = *reinterpret_cast<const f32x4_t*>(a.rh + idx * 4);
    float pre[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const long long off = (long long)(g * N + n) * D + u;
      pre[g] = rh[g] + ld_f(a.Wx, wbase + off, a.wx_f32) + (a.bias ? ld_f(a.bias, off, rf) : 0.0f);
    }
    const float ig = sigmoid_f(pre[0]), fg = sigmoid_f(pre[1]), zg = tanh_f(pre[2]), og = sigmoid_f(pre[3]);
    c = fg * a.ccur[idx] + ig * zg;
    a.ccur[idx] = c;
    h = og * tanh_f(c);
  } else if (a.cell == CELL_GRU) {
    // the reset gate scales the candidate's recurrent part (h.R_n + b_n), not its Wx
    const f32x4_t rh = *reinterpret_cast<const f32x4_t*>(a.rh + idx * 4);
    float wx[3], bb[3];
#pragma unroll
    for (int g = 0; g < 3; ++g) {
      const long long off = (long long)(g * N + n) * D + u;
      wx[g] = ld_f(a.Wx, wbase + off, a.wx_f32);
      bb[g] = a.bias ? ld_f(a.bias, off, rf) : 0.0f;
    }
    const float rg = sigmoid_f(rh[0] + wx[0] + bb[0]);
    const float zg = sigmoid_f(rh[1] + wx[1] + bb[1]);
    const float ng = tanh_f(wx[2] + rg * (rh[2] + bb[2]));
    h = ng + zg * (a.ccur[idx] - ng);  // (1 - z) n + z h
    a.ccur[idx] = h;
  } else {
    const long long off = (long long)n * D + u;
    h = tanh_f(a.rh[idx] + ld_f(a.Wx, wbase + off, a.wx_f32) + (a.bias ? ld_f(a.bias, off, rf) : 0.0f));
  }
  if (a.out_h) a.out_h[o] = h;
  if (a.out_c && a.cell == CELL_LSTM) a.out_c[o] = c;
  if (t == a.T - 1) {
    const long long lo = b * a.last_sb + (long long)n * a.last_sn + u;
    if (a.last_h) a.last_h[lo] = h;
    if (a.last_c && a.cell == CELL_LSTM) a.last_c[lo] = c;
  }
  const long long hi = ((long long)n * a.B + b) * D + u;
  if (rf) reinterpret_cast<float*>(a.hcur)[hi] = h;
  else reinterpret_cast<uint16_t*>(a.hcur)[hi] = f2bf(h);
}

}  // namespace frnn
