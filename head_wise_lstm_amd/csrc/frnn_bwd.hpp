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
//      that reaches h_{t-1}, dh = sum_g da_g . R_g^T, in BWD_KS parts over K that the next
//      pointwise kernel adds;
//   3. dR = sum over (t, b) of h_{t-1}^T da, one GEMM per head over K = T*B, with db from a row of
//      ones appended to h^T.
// Operands of the contractions are bf16 (fp32 for fp32 inputs) with fp32 accumulation, like the
// forward; every carried gradient and every output is fp32.
#pragma once

#include <type_traits>

#include "frnn_device.hpp"

namespace frnn {

struct BwdArgs {
  int B, T, N, D, cell;
  int f32;        // operands fp32 (else bf16): R, bias, initial states, the MFMA operands
  int wx_f32;     // Wx fp32 (else bf16)
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
  const void* rpk;    // R packed as the dh kernel's A fragments (bwd_rpack_kernel)
  float* dhpart;      // [BWD_KS][B][N][D]: K-split parts of the gradient reaching h through R
  int ks;             // parts in use (<= BWD_KS)
  float* carry;       // [B][N][D]: LSTM dc, GRU direct dh carried to the step before
  const float* zeros; // 256 zero bytes: absent inputs read element 0 of it, so no load is conditional
};

constexpr int BWD_KS = 4;  // K split of the dh kernel

__device__ __forceinline__ void st_op(void* p, long long i, float v, bool f32) {
  if (f32) reinterpret_cast<float*>(p)[i] = v;
  else reinterpret_cast<uint16_t*>(p)[i] = f2bf(v);
}

// hprev[n][t*B + b][d] = h_{t-1}[b][n][d] (the initial state for t = 0), in the operand type;
// rows T*B .. Kp-1 are zero.
// Eight consecutive d per thread (D is a multiple of 32): the index arithmetic once per eight
// elements, and one 16-byte store of the bf16 operand (two of fp32).
__global__ void __launch_bounds__(256) bwd_hprev_kernel(BwdArgs a) {
  const int DC = a.D / 8;
  const long long total = (long long)a.N * a.Kp * DC;
  const bool f32 = a.f32;
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (long long)gridDim.x * 256) {
    const int d0 = (int)(idx % DC) * 8;
    const long long r = idx / DC;
    const int row = (int)(r % a.Kp);
    const int n = (int)(r / a.Kp);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    if (row < a.T * a.B) {
      const int t = row / a.B, b = row % a.B;
      if (t > 0) {
        const float* src = a.st_h + (long long)b * a.st_sb + (long long)(t - 1) * a.st_st + (long long)n * a.D + d0;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = src[i];
      } else if (a.s0_h) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = ld_f(a.s0_h, (long long)b * a.s0_sb + (long long)n * a.D + d0 + i, f32);
      }
    }
    const long long o = r * a.D + d0;  // element index of the operand
    if (f32) {
      float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.hprev) + o);
      dst[0] = make_float4(v[0], v[1], v[2], v[3]);
      dst[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
      uint4 w;
      w.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
      w.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
      w.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
      w.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.hprev) + o) = w;
    }
  }
}

// The dR GEMM's A operand straight from the states, bf16: hT[n][d][k] = h_{t-1}[b][n][d] for k = t*B
// + b < T*B (the initial state, or zero, for t = 0), zero for k up to Kp (row d = D, the ones, is
// bwd_ones_row_kernel's). 64 k x 64 d tiles through LDS: each row of a tile is read as 256 bytes
// of fp32 (16-byte loads), and each output row written as 128 bytes (8-byte stores). Grid
// (ceil(D / 64), min(Kp / 64, 65535), N), the k tiles repeating by gridDim.y; D a multiple of 32
// (a tile's rows past D stay empty). Where the h.R recompute is not needed this replaces
// bwd_hprev_kernel and the transpose of its output.
__global__ void __launch_bounds__(256) bwd_hprevT_kernel(BwdArgs a, uint16_t* hT) {
  __shared__ __attribute__((aligned(16))) uint16_t s[64][68];
  const int d0 = blockIdx.x * 64, n = blockIdx.z;
  const int D = a.D, TB = a.T * a.B;
  const int t16 = threadIdx.x >> 4, c4 = (threadIdx.x & 15) * 4;  // row t16 + 16 i, 4 d from c4
  for (int kb = blockIdx.y; kb * 64 < a.Kp; kb += gridDim.y) {
    const int k0 = kb * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = k0 + t16 + 16 * i, d = d0 + c4;
      float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (k < TB && d < D) {
        const int t = k / a.B, b = k - t * a.B;
        if (t > 0) {
          const f32x4_t x = *reinterpret_cast<const f32x4_t*>(a.st_h + (long long)b * a.st_sb + (long long)(t - 1) * a.st_st +
                                                           (long long)n * D + d);
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = x[q];
        } else if (a.s0_h) {
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = ld_f(a.s0_h, (long long)b * a.s0_sb + (long long)n * D + d + q, false);
        }
      }
      uint2 w;
      w.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
      w.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
      *reinterpret_cast<uint2*>(&s[t16 + 16 * i][c4]) = w;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = t16 + 16 * i, d = d0 + j;  // output row d, 4 k from k0 + c4
      if (d >= D) continue;
      uint2 w;
      w.x = (uint32_t)s[c4][j] | ((uint32_t)s[c4 + 1][j] << 16);
      w.y = (uint32_t)s[c4 + 2][j] | ((uint32_t)s[c4 + 3][j] << 16);
      *reinterpret_cast<uint2*>(hT + ((long long)n * (D + 1) + d) * a.Kp + k0 + c4) = w;
    }
    __syncthreads();
  }
}

// The coefficients of step t for one (b, n, unit): everything the backward of the step needs
// that does not depend on the gradient arriving from later steps (the gates from the recomputed
// h.R, Wx and the bias, the states, and the gradients of the step's own outputs). The record
// layout (two f32x4) is the fused serial part's (frnn_fused_bwd.hpp):
//   LSTM: r0 = (o tanh'(c), z i', c_prev f', i z'), r1 = (tanh(c) o', f, dstates_h, dstates_c)
//   GRU:  r0 = (c3 q r', (h_prev - n) z', c3 r, z), r1 = (dstates_h, c3), c3 = (1 - z) n'
//   Elman: r0 = (1 - h^2, dstates_h)
// (x' the derivative of the gate's nonlinearity at its value; dstates includes last_states'
// gradient at t = T-1).
template <int CELL, bool F32, bool WXF32>
__device__ __forceinline__ void bwd_coeffs(const BwdArgs& a, int t, int b, int n, int u, f32x4_t& r0, f32x4_t& r1) {
  constexpr int G = cell_gates(CELL);
  typedef typename std::conditional<F32, float, uint16_t>::type op_t;
  typedef typename std::conditional<WXF32, float, uint16_t>::type wx_t;
  const int N = a.N, D = a.D;
  const long long tb = (long long)t * a.B + b;
  const float* hr = a.hr + ((long long)n * a.T * a.B + tb) * G * D + u;
  const long long wbase = (long long)b * a.wx_sb + (long long)t * a.wx_st + (long long)n * D + u;
  const long long sidx = (long long)b * a.st_sb + (long long)t * a.st_st + (long long)n * D + u;
  const long long lidx = (long long)b * a.last_sb + (long long)n * D + u;
  const long long s0idx = (long long)b * a.s0_sb + (long long)n * D + u;
  // every input is read unconditionally: an absent one (or one this step does not use) is read
  // at element 0 of the zero page instead
  const op_t* zop = reinterpret_cast<const op_t*>(a.zeros);
  const wx_t* wxp = reinterpret_cast<const wx_t*>(a.Wx);
  const bool hb = a.bias != nullptr, hds = a.ds_h != nullptr, hdl = a.dl_h != nullptr && t == a.T - 1;
  const op_t* bp = hb ? reinterpret_cast<const op_t*>(a.bias) : zop;
  const float* dsh = hds ? a.ds_h : a.zeros;
  const float* dlh = hdl ? a.dl_h : a.zeros;
  auto f = [](op_t v) -> float {
    if constexpr (F32) return v;
    else return bf2f(v);
  };
  auto fw = [](wx_t v) -> float {
    if constexpr (WXF32) return v;
    else return bf2f(v);
  };
  float pre[G], wx[G], bb[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    pre[g] = hr[(long long)g * D];
    wx[g] = fw(wxp[wbase + (long long)g * N * D]);
    bb[g] = f(bp[hb ? (long long)(g * N + n) * D + u : 0]);
  }
  const float ds_h = dsh[hds ? sidx : 0] + dlh[hdl ? lidx : 0];
  if constexpr (CELL == CELL_LSTM) {
    const bool hdc = a.ds_c != nullptr, hlc = a.dl_c != nullptr && t == a.T - 1, hs0 = a.s0_c != nullptr;
    const float* dsc = hdc ? a.ds_c : a.zeros;
    const float* dlc = hlc ? a.dl_c : a.zeros;
    const op_t* s0c = hs0 ? reinterpret_cast<const op_t*>(a.s0_c) : zop;
    const float ct = a.st_c[sidx];
    const float cprev = a.st_c[t > 0 ? sidx - a.st_st : sidx];
    const float c0 = f(s0c[hs0 ? s0idx : 0]);
    const float cp = t > 0 ? cprev : c0;
    const float ds_c = dsc[hdc ? sidx : 0] + dlc[hlc ? lidx : 0];
    const float ig = sigmoid_f(pre[0] + wx[0] + bb[0]);
    const float fg = sigmoid_f(pre[1] + wx[1] + bb[1]);
    const float zg = tanh_f(pre[2] + wx[2] + bb[2]);
    const float og = sigmoid_f(pre[3] + wx[3] + bb[3]);
    const float tc = tanh_f(ct);
    r0 = f32x4_t{og * (1.0f - tc * tc), zg * ig * (1.0f - ig), cp * fg * (1.0f - fg), ig * (1.0f - zg * zg)};
    r1 = f32x4_t{tc * og * (1.0f - og), fg, ds_h, ds_c};
  } else if constexpr (CELL == CELL_GRU) {
    const bool hs0 = a.s0_h != nullptr;
    const op_t* s0h = hs0 ? reinterpret_cast<const op_t*>(a.s0_h) : zop;
    const float hprev = a.st_h[t > 0 ? sidx - a.st_st : sidx];
    const float h0 = f(s0h[hs0 ? s0idx : 0]);
    const float hp = t > 0 ? hprev : h0;
    const float rg = sigmoid_f(pre[0] + wx[0] + bb[0]);
    const float zg = sigmoid_f(pre[1] + wx[1] + bb[1]);
    const float q = pre[2] + bb[2];
    const float ng = tanh_f(wx[2] + rg * q);
    const float c3 = (1.0f - zg) * (1.0f - ng * ng);
    r0 = f32x4_t{c3 * q * rg * (1.0f - rg), (hp - ng) * zg * (1.0f - zg), c3 * rg, zg};
    r1 = f32x4_t{ds_h, c3, 0.0f, 0.0f};
  } else {
    const float ht = a.st_h[sidx];
    r0 = f32x4_t{1.0f - ht * ht, ds_h, 0.0f, 0.0f};
    r1 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
}

// Coefficient records of every step, for the fused serial part: one thread per (t, b, n, unit);
// record index s = T-1-t. REC floats a record: 8 (both f32x4), or 2 for an Elman cell, whose
// record is r0's first two (the single-workgroup design's compact records).
template <int CELL, bool F32, bool WXF32, int REC = 8>
__global__ void __launch_bounds__(256) bwd_record_kernel(BwdArgs a, float* rec) {
  static_assert(REC == 8 || (REC == 2 && CELL == CELL_ELMAN), "compact records hold an Elman cell's two coefficients");
  const long long total = (long long)a.T * a.B * a.N * a.D;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int u = (int)(idx % a.D);
  long long r = idx / a.D;
  const int n = (int)(r % a.N);
  r /= a.N;
  const int b = (int)(r % a.B);
  const int t = (int)(r / a.B);
  f32x4_t r0, r1;
  bwd_coeffs<CELL, F32, WXF32>(a, t, b, n, u, r0, r1);
  const long long s = (long long)(a.T - 1 - t);
  const long long ri = ((s * a.B + b) * a.N + n) * a.D + u;
  if constexpr (REC == 2) {
    reinterpret_cast<float2*>(rec)[ri] = make_float2(r0[0], r0[1]);
  } else {
    f32x4_t* out = reinterpret_cast<f32x4_t*>(rec + ri * 8);
    out[0] = r0;
    out[1] = r1;
  }
}

// The gradients of step t for one (b, n, unit) from its coefficients and the gradients reaching
// its state: dh (h_t) and, for the LSTM, dc (c_t, everything included). Writes dWx and the dR
// operand da; returns the gradient carried to step t-1 past R (LSTM: dc . f; GRU: dh . z; Elman: 0).
template <int CELL, bool F32>
__device__ __forceinline__ float bwd_apply(const BwdArgs& a, int t, int b, int n, int u, f32x4_t r0, f32x4_t r1,
                                           float dh, float dc) {
  constexpr int G = cell_gates(CELL);
  const int N = a.N, D = a.D;
  float dw[G], dav[G];
  float carry = 0.0f;
  if constexpr (CELL == CELL_LSTM) {
    dw[0] = dc * r0[1];
    dw[1] = dc * r0[2];
    dw[2] = dc * r0[3];
    dw[3] = dh * r1[0];
    carry = dc * r1[1];
#pragma unroll
    for (int g = 0; g < 4; ++g) dav[g] = dw[g];
  } else if constexpr (CELL == CELL_GRU) {
    dw[0] = dh * r0[0];
    dw[1] = dh * r0[1];
    dw[2] = dh * r1[1];
    dav[0] = dw[0];
    dav[1] = dw[1];
    dav[2] = dh * r0[2];
    carry = dh * r0[3];
  } else {
    dw[0] = dh * r0[0];
    dav[0] = dw[0];
  }
  const long long wbase = (long long)b * a.wx_sb + (long long)t * a.wx_st + (long long)n * D + u;
  if (a.dWx) {
#pragma unroll
    for (int g = 0; g < G; ++g) a.dWx[wbase + (long long)g * N * D] = dw[g];
  }
  const long long drow = ((long long)n * a.Kp + (long long)t * a.B + b) * G * D + u;
#pragma unroll
  for (int g = 0; g < G; ++g) st_op(a.da, drow + (long long)g * D, dav[g], F32);
  return carry;
}

// dWx, the dR operand da and (at t = 0) the carries from the fused serial part's (dh, dc) and the
// records: one thread per (t, b, n, unit).
template <int CELL, bool F32>
__global__ void __launch_bounds__(256) bwd_post_kernel(BwdArgs a, const float* rec, const float* dstate) {
  const long long total = (long long)a.T * a.B * a.N * a.D;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int u = (int)(idx % a.D);
  long long r = idx / a.D;
  const int n = (int)(r % a.N);
  r /= a.N;
  const int b = (int)(r % a.B);
  const int t = (int)(r / a.B);
  const int N = a.N, D = a.D;
  const long long s = (long long)(a.T - 1 - t);
  const long long ri = ((s * a.B + b) * N + n) * D + u;
  const f32x4_t r0 = reinterpret_cast<const f32x4_t*>(rec)[ri * 2];
  const f32x4_t r1 = reinterpret_cast<const f32x4_t*>(rec)[ri * 2 + 1];
  const float2 st = reinterpret_cast<const float2*>(dstate)[ri];
  const float carry = bwd_apply<CELL, F32>(a, t, b, n, u, r0, r1, st.x, st.y);
  if (t == 0) a.carry[((long long)b * N + n) * D + u] = carry;
}

// Step t of the alternating serial part, one thread per (b, n, unit), consecutive threads on
// consecutive units: the gradient reaching h_t through R (the K-split parts that step t+1's
// bwd_dh_kernel left in dhpart) plus the step's own, then the step's coefficients (bwd_coeffs) and
// gradients (bwd_apply): dWx, da and the carry.
template <int CELL, bool F32, bool WXF32>
__global__ void __launch_bounds__(64) bwd_gate_kernel(BwdArgs a, int t) {
  const long long total = (long long)a.B * a.N * a.D;
  const long long idx = (long long)blockIdx.x * 64 + threadIdx.x;
  if (idx >= total) return;
  const int u = (int)(idx % a.D);
  const long long r = idx / a.D;
  const int n = (int)(r % a.N);
  const int b = (int)(r / a.N);
  const long long BND = total;
  float dp[BWD_KS];
#pragma unroll
  for (int k = 0; k < BWD_KS; ++k) dp[k] = a.dhpart[(k < a.ks ? k * BND : 0) + idx];
  const float cin = CELL != CELL_ELMAN ? a.carry[idx] : 0.0f;
  f32x4_t r0, r1;
  bwd_coeffs<CELL, F32, WXF32>(a, t, b, n, u, r0, r1);
  float dhr = 0.0f;
#pragma unroll
  for (int k = 0; k < BWD_KS; ++k) dhr += k < a.ks ? dp[k] : 0.0f;
  float dh, dc = 0.0f;
  if constexpr (CELL == CELL_LSTM) {
    dh = dhr + r1[2];
    dc = cin + r1[3] + dh * r0[0];
  } else if constexpr (CELL == CELL_GRU) {
    dh = dhr + r1[0] + cin;
  } else {
    dh = dhr + r0[1];
  }
  const float carry = bwd_apply<CELL, F32>(a, t, b, n, u, r0, r1, dh, dc);
  if (CELL != CELL_ELMAN) a.carry[idx] = carry;
}

// Step t of the alternating serial part in one launch: the contraction dhr = da_{t+1} . R^T for
// one 16-unit tile of d and 16 batch columns (grid (D/16, 1, ceil(B/16)*N); skipped at t = T-1,
// where nothing reaches h through R), then, as its epilogue, the step's backward for the tile's 16
// units of the 16 batch columns (bwd_coeffs, then bwd_apply). The tile's result puts units
// 4*(l/16)..+3 of batch column l%16 in lane l. The 16 waves take the k-tiles of K = G*D 16 apart,
// issue all of a batch of fragment loads before its MFMAs, and meet in LDS. da_{t+1} and da_t are
// different rows of the da buffer, and each carry belongs to one lane, so no workgroup overwrites
// what another of the same launch still reads.
//
// Against bwd_gate_kernel + bwd_dh_kernel (two launches per step) it trades a launch for a whole K
// of R and da per workgroup (G*D*64 bytes): the planner takes it where G*D <= 1024 (ms per call,
// one launch / two: LSTM B=8 N=3 D=256 6.02 / 7.69, Elman B=64 N=12 D=64 14.44 / 16.94, LSTM fp32
// D=32 0.119 / 0.148), and the two launches above (LSTM D=768 9.80 / 7.85, GRU D=768 8.05 / 7.50,
// the two-layer LSTM's H=512 14.57 / 14.25).
constexpr int BWD_STEP_WAVES = 16;

template <int CELL, bool F32, bool WXF32>
__global__ void __launch_bounds__(BWD_STEP_WAVES * 64) bwd_step_kernel(BwdArgs a, int t) {
  constexpr int NW = BWD_STEP_WAVES;
  __shared__ f32x4_t part[NW][64];
  constexpr int G = cell_gates(CELL);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, quad = lane >> 4;
  const int D = a.D;
  const int dt = blockIdx.x;
  const int nbb = (a.B + 15) / 16;
  const int n = blockIdx.z / nbb, b0 = (blockIdx.z % nbb) * 16;
  const bool colv = b0 + col < a.B;
  // the epilogue's inputs first (waves 0-3, unit 4*(l/16) + wave of lane l): they do not depend on
  // the contraction, so their loads and transcendentals overlap it
  const bool epi = wave < 4 && colv;
  const int ue = dt * 16 + 4 * quad + (wave & 3);
  const long long cidx = ((long long)(b0 + col) * a.N + n) * D + ue;
  f32x4_t r0 = {0.f, 0.f, 0.f, 0.f}, r1 = {0.f, 0.f, 0.f, 0.f};
  float cin = 0.0f;
  if (epi) {
    bwd_coeffs<CELL, F32, WXF32>(a, t, b0 + col, n, ue, r0, r1);
    if (CELL != CELL_ELMAN) cin = a.carry[cidx];
  }
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  if (t + 1 < a.T) {
    constexpr int KW = F32 ? 4 : 32;
    constexpr int KB = F32 ? 16 : 8;
    typedef typename std::conditional<F32, float, bf16x8_t>::type frag_t;
    const int KT = G * D / KW;
    const long long drow = ((long long)n * a.Kp + (long long)(t + 1) * a.B + b0 + col) * G * D;
    const long long rbase = (((long long)n * (D / 16) + dt) * KT) * 64 + lane;
    for (int k0 = wave; k0 < KT; k0 += NW * KB) {
      frag_t ra[KB], db[KB];
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const int k = k0 + NW * j;
        const bool kv = k < KT;
        if constexpr (F32) {
          ra[j] = kv ? reinterpret_cast<const float*>(a.rpk)[rbase + (long long)k * 64] : 0.0f;
          db[j] = (kv && colv) ? reinterpret_cast<const float*>(a.da)[drow + k * KW + quad] : 0.0f;
        } else {
          u32x4_t rv = {0u, 0u, 0u, 0u}, dv = {0u, 0u, 0u, 0u};
          if (kv) rv = reinterpret_cast<const u32x4_t*>(a.rpk)[rbase + (long long)k * 64];
          if (kv && colv) dv = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(a.da) + drow + k * KW + 8 * quad);
          ra[j] = __builtin_bit_cast(bf16x8_t, rv);
          db[j] = __builtin_bit_cast(bf16x8_t, dv);
        }
      }
#pragma unroll
      for (int j = 0; j < KB; j += 2) {
        if (k0 + NW * j >= KT) break;  // (uniform in the wave)
        if constexpr (F32) {
          acc0 = mfma_f32(ra[j], db[j], acc0);
          acc1 = mfma_f32(ra[j + 1], db[j + 1], acc1);
        } else {
          acc0 = mfma_bf16(ra[j], db[j], acc0);
          acc1 = mfma_bf16(ra[j + 1], db[j + 1], acc1);
        }
      }
    }
  }
  part[wave][lane] = acc0 + acc1;
  __syncthreads();
  // the epilogue: wave i < 4 takes unit 4*(l/16) + i of lane l, so that a lane's loads and stores
  // are those of one element (one lane handling four units in turn would wait for each unit's
  // stores before the next unit's loads: on gfx9 a wave's memory counter retires both in order)
  if (!epi) return;
  float dhr = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) dhr += reinterpret_cast<const float*>(&part[w][lane])[wave];
  float dh, dc = 0.0f;
  if constexpr (CELL == CELL_LSTM) {
    dh = dhr + r1[2];
    dc = cin + r1[3] + dh * r0[0];
  } else if constexpr (CELL == CELL_GRU) {
    dh = dhr + r1[0] + cin;
  } else {
    dh = dhr + r0[1];
  }
  const float carry = bwd_apply<CELL, F32>(a, t, b0 + col, n, ue, r0, r1, dh, dc);
  if (CELL != CELL_ELMAN) a.carry[cidx] = carry;
}

// R in the dh kernel's A-fragment order: [N][D/16 row tiles][G*D/KW k-tiles][64 lanes] x (8 bf16
// | 1 fp32); lane (m, quad) of tile (dt, kt) holds R[g][n][16 dt + m][e0 + 8 quad ..] (bf16) or
// [e0 + quad] (fp32), with (g, e0) the k-tile's gate and first unit. One thread per lane entry.
__global__ void __launch_bounds__(256) bwd_rpack_kernel(BwdArgs a, void* out) {
  const int G = cell_gates(a.cell), D = a.D;
  const int KW = a.f32 ? 4 : 32;
  const int KT = G * D / KW, DT = D / 16;
  const long long total = (long long)a.N * DT * KT * 64;
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (long long)gridDim.x * 256) {
    const int lane = (int)(idx & 63);
    long long r = idx >> 6;
    const int kt = (int)(r % KT);
    r /= KT;
    const int dt = (int)(r % DT);
    const int n = (int)(r / DT);
    const int m = lane & 15, quad = lane >> 4;
    const int g = kt * KW / D, e0 = kt * KW % D;
    const long long row = (long long)g * a.r_sg + (long long)n * a.r_sn + (long long)(dt * 16 + m) * a.r_sd + e0;
    if (a.f32) {
      reinterpret_cast<float*>(out)[idx] = reinterpret_cast<const float*>(a.R)[row + quad];
    } else {
      reinterpret_cast<u32x4_t*>(out)[idx] =
          *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(a.R) + row + 8 * quad);
    }
  }
}

// dh of step t-1, part ks of the K split: dhpart[ks][b][n][d] = sum over k-tiles kt of this part
// of sum_e da[n][t*B + b][k] * R[g][n][d][e] (k = (g, e)). MFMA with A = packed R (16 values of
// d, 1 KiB per wave-load) and B = da^T (batch in the 16 columns). Grid (D/16, ks, ceil(B/16)*N);
// the 4 waves take the part's k-tiles 4 apart and meet in LDS.
template <bool F32>
__global__ void __launch_bounds__(256) bwd_dh_kernel(BwdArgs a, int t) {
  __shared__ f32x4_t part[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, quad = lane >> 4;
  const int G = cell_gates(a.cell), D = a.D;
  const int dt = blockIdx.x, ks = blockIdx.y;
  const int nbb = (a.B + 15) / 16;
  const int n = blockIdx.z / nbb, b0 = (blockIdx.z % nbb) * 16;
  const int KW = F32 ? 4 : 32;
  const int KT = G * D / KW;
  const int k_lo = (int)((long long)KT * ks / a.ks), k_hi = (int)((long long)KT * (ks + 1) / a.ks);
  const bool colv = b0 + col < a.B;
  const long long drow = ((long long)n * a.Kp + (long long)t * a.B + b0 + col) * G * D;
  const long long rbase = (((long long)n * (D / 16) + dt) * KT) * 64 + lane;
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  int k = k_lo + wave;
  for (; k + 4 < k_hi; k += 8) {
    if constexpr (F32) {
      const float* rp = reinterpret_cast<const float*>(a.rpk) + rbase;
      const float* dp = reinterpret_cast<const float*>(a.da) + drow + quad;
      const float a0 = rp[(long long)k * 64], a1 = rp[(long long)(k + 4) * 64];
      const float h0 = colv ? dp[k * KW] : 0.0f, h1 = colv ? dp[(k + 4) * KW] : 0.0f;
      acc0 = mfma_f32(a0, h0, acc0);
      acc1 = mfma_f32(a1, h1, acc1);
    } else {
      const u32x4_t* rp = reinterpret_cast<const u32x4_t*>(a.rpk) + rbase;
      const uint16_t* dp = reinterpret_cast<const uint16_t*>(a.da) + drow + 8 * quad;
      const u32x4_t a0 = rp[(long long)k * 64], a1 = rp[(long long)(k + 4) * 64];
      u32x4_t h0 = {0u, 0u, 0u, 0u}, h1 = {0u, 0u, 0u, 0u};
      if (colv) {
        h0 = *reinterpret_cast<const u32x4_t*>(dp + k * KW);
        h1 = *reinterpret_cast<const u32x4_t*>(dp + (k + 4) * KW);
      }
      acc0 = mfma_bf16(__builtin_bit_cast(bf16x8_t, a0), __builtin_bit_cast(bf16x8_t, h0), acc0);
      acc1 = mfma_bf16(__builtin_bit_cast(bf16x8_t, a1), __builtin_bit_cast(bf16x8_t, h1), acc1);
    }
  }
  if (k < k_hi) {
    if constexpr (F32) {
      const float a0 = reinterpret_cast<const float*>(a.rpk)[rbase + (long long)k * 64];
      const float h0 = colv ? reinterpret_cast<const float*>(a.da)[drow + k * KW + quad] : 0.0f;
      acc0 = mfma_f32(a0, h0, acc0);
    } else {
      const u32x4_t a0 = reinterpret_cast<const u32x4_t*>(a.rpk)[rbase + (long long)k * 64];
      u32x4_t h0 = {0u, 0u, 0u, 0u};
      if (colv) h0 = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(a.da) + drow + k * KW + 8 * quad);
      acc0 = mfma_bf16(__builtin_bit_cast(bf16x8_t, a0), __builtin_bit_cast(bf16x8_t, h0), acc0);
    }
  }
  part[wave][lane] = acc0 + acc1;
  __syncthreads();
  if (wave != 0 || !colv) return;
  const f32x4_t s = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
  const long long BND = (long long)a.B * a.N * D;
  *reinterpret_cast<f32x4_t*>(a.dhpart + ks * BND + ((long long)(b0 + col) * a.N + n) * D + dt * 16 + 4 * quad) = s;
}

// dstates0 from what reaches the initial state: h through R (plus the GRU's direct part), and
// the LSTM's carried dc.
__global__ void __launch_bounds__(256) bwd_final_kernel(BwdArgs a) {
  const long long total = (long long)a.B * a.N * a.D;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const long long BND = (long long)a.B * a.N * a.D;
  float dh = a.cell == CELL_GRU ? a.carry[idx] : 0.0f;
  for (int k = 0; k < a.ks; ++k) dh += a.dhpart[k * BND + idx];
  if (a.ds0_h) a.ds0_h[idx] = dh;
  if (a.ds0_c && a.cell == CELL_LSTM) a.ds0_c[idx] = a.carry[idx];
}

// dR[g][n][d][e] (element strides dr_sg, dr_sn, dr_sd; e contiguous) = sum_p tmp[p][n][d][g*D + e]
// and db[g][n][e] = sum_p tmp[p][n][D][g*D + e]
// (tmp: [parts][N][D+1][G*D] fp32, the K-split parts of the dR GEMM's output with its row of
// ones), the parts added in order.
// Four consecutive e per thread (one 16-byte load of each part; D is a multiple of 32, so the
// four stay in one gate).
__global__ void __launch_bounds__(256) bwd_scatter_kernel(const float* tmp, int parts, int N, int D, int G, float* dR,
                                                          long long dr_sg, long long dr_sn, long long dr_sd, float* db) {
  const long long total = (long long)N * (D + 1) * G * D;
  const int CPR = G * D / 4;  // chunks of four per row
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < total / 4; idx += (long long)gridDim.x * 256) {
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < parts; ++p) v += *reinterpret_cast<const f32x4_t*>(tmp + p * total + 4 * idx);
    const int col = (int)(idx % CPR) * 4;
    const long long r = idx / CPR;
    const int d = (int)(r % (D + 1));
    const int n = (int)(r / (D + 1));
    const int g = col / D, e = col % D;
    if (d < D) {
      if (dR) {
        float* o = dR + (long long)g * dr_sg + (long long)n * dr_sn + (long long)d * dr_sd + e;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = v[i];
      }
    } else if (db) {
      float* o = db + ((long long)g * N + n) * D + e;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = v[i];
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
                                                       const float* Bt, long long ldb, float* C, long long ldc,
                                                       long long a_z, long long b_z, long long c_z, long long a_h,
                                                       long long b_h, long long c_h) {
  A += blockIdx.y * a_z + blockIdx.z * a_h;  // part blockIdx.y of head blockIdx.z of a batch of products
  Bt += blockIdx.y * b_z + blockIdx.z * b_h;
  C += blockIdx.y * c_z + blockIdx.z * c_h;
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
