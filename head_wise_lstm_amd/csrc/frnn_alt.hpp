// Alternating forward recurrence for gfx950: per step one launch, the MFMA contraction h.R for
// all heads and batch rows with the gates as its epilogue; the step's synchronisation is the
// kernel boundary, and R is re-read (from L2) every step, so any head size runs. R is packed once
// per call into MFMA-fragment order, so every per-step operand load is a contiguous 1 KiB per wave.
// h alternates between two buffers: step t reads one and writes the other, so a workgroup that
// has finished its units cannot overwrite h that another workgroup of the same step still reads.
//
// Tiles follow the fused design: a 16-row tile of R^T holds the four gate rows of four units
// (LSTM; GRU with a zero fourth row) or sixteen units (Elman); lane l of the MFMA result holds
// rows 4*(l/16)+i of batch column l%16, so after the K split's sum a lane holds every gate of its
// unit (or four units of the Elman cell) and gates without cross-lane traffic.
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
  void* hbuf[2];  // h, MFMA operand type, [N][B][D] each: step t reads hbuf[t & 1], writes the other
  float* ccur;    // current c (LSTM) or h in fp32 (GRU): [B][N][D]
};

// Initial state into the working buffers: hbuf[0][n][b][d] (operand type), ccur[b][n][d] (the
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
    if (a.r_is_f32) reinterpret_cast<float*>(a.hbuf[0])[hi] = h;
    else reinterpret_cast<uint16_t*>(a.hbuf[0])[hi] = f2bf(h);
    a.ccur[idx] = c;
  }
}

// Step t: grid (TPH, ceil(B/16), N), one R^T tile per workgroup. The 4 waves take the tile's
// k-tiles 4 apart (wave w: w, w+4, ...), each with two accumulators and all its loads in flight at
// once; the four partial sums meet in LDS, and wave 0 adds Wx and the bias (loaded before the
// contraction), applies the gates and writes the step's states.
template <bool F32>
__global__ void __launch_bounds__(256) alt_step_kernel(AltArgs a, int t) {
  __shared__ f32x4_t part[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, quad = lane >> 4;
  const int GS = cell_slots(a.cell);
  const int N = a.N, D = a.D;
  const int TPH = GS * D / 16;
  const int tt = blockIdx.x;
  const int b0 = blockIdx.y * 16;
  const int n = blockIdx.z;
  const int KW = F32 ? 4 : 32;
  const int KT = D / KW;
  const bool colv = b0 + col < a.B;
  const void* hin = a.hbuf[t & 1];
  void* hout = a.hbuf[(t + 1) & 1];
  const bool rf = F32;

  // ---- the epilogue's inputs (wave 0): Wx, bias and the carried state do not depend on h, so
  // their loads go out first and their latency hides behind the contraction's
  const long long b = b0 + col;
  const int ts = n >= a.rev_n0 ? a.T - 1 - t : t;  // the head's time direction
  const long long wbase = b * a.wx_sb + (long long)ts * a.wx_st;
  const long long sbase = (b * N + n) * D;  // ccur
  const int ue = GS == 4 ? 4 * tt + quad : 16 * tt + 4 * quad;  // the lane's (first) unit
  float pin[4] = {0.f, 0.f, 0.f, 0.f}, cprev = 0.0f;  // Wx + bias per gate (LSTM, GRU) or unit (Elman)
  float bn = 0.0f;                                    // GRU: the candidate's bias, added inside r (.)
  if (wave == 0 && colv) {
    if (GS == 4) {
      const int G = cell_gates(a.cell);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (g >= G) continue;
        const long long off = (long long)(g * N + n) * D + ue;
        const float bb = a.bias ? ld_f(a.bias, off, rf) : 0.0f;
        const float wx = ld_f(a.Wx, wbase + off, a.wx_f32);
        if (a.cell == CELL_GRU && g == 2) { pin[g] = wx; bn = bb; }
        else pin[g] = wx + bb;
      }
      cprev = a.ccur[sbase + ue];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long long off = (long long)n * D + ue + i;
        pin[i] = ld_f(a.Wx, wbase + off, a.wx_f32) + (a.bias ? ld_f(a.bias, off, rf) : 0.0f);
      }
    }
  }

  // ---- the contraction: wave w takes k-tiles w, w+4, ...; all of a batch of KB k-tiles' loads
  // (R fragments and h) go out before the first MFMA, so the wave waits for memory once per batch
  // (one batch for every bf16 head up to D = 1024)
  constexpr int KB = F32 ? 16 : 8;
  typedef typename std::conditional<F32, float, bf16x8_t>::type frag_t;
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = wave; k0 < KT; k0 += 4 * KB) {
    frag_t ra[KB], hb[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int kt = k0 + 4 * j;
      const bool kv = kt < KT;
      if constexpr (F32) {
        const float* rp = reinterpret_cast<const float*>(a.rpack) + ((long long)n * TPH + tt) * KT * 64 + lane;
        const float* hp = reinterpret_cast<const float*>(hin) + ((long long)n * a.B + b0 + col) * D + quad;
        ra[j] = kv ? rp[(long long)kt * 64] : 0.0f;
        hb[j] = (kv && colv) ? hp[kt * 4] : 0.0f;
      } else {
        const u32x4_t* rp = reinterpret_cast<const u32x4_t*>(a.rpack) + ((long long)n * TPH + tt) * KT * 64 + lane;
        const uint16_t* hp = reinterpret_cast<const uint16_t*>(hin) + ((long long)n * a.B + b0 + col) * D + 8 * quad;
        u32x4_t rv = {0u, 0u, 0u, 0u}, hv = {0u, 0u, 0u, 0u};
        if (kv) rv = rp[(long long)kt * 64];
        if (kv && colv) hv = *reinterpret_cast<const u32x4_t*>(hp + kt * 32);
        ra[j] = __builtin_bit_cast(bf16x8_t, rv);
        hb[j] = __builtin_bit_cast(bf16x8_t, hv);
      }
    }
#pragma unroll
    for (int j = 0; j < KB; j += 2) {
      if (k0 + 4 * j >= KT) break;  // (uniform in the wave)
      if constexpr (F32) {
        acc0 = mfma_f32(ra[j], hb[j], acc0);
        acc1 = mfma_f32(ra[j + 1], hb[j + 1], acc1);
      } else {
        acc0 = mfma_bf16(ra[j], hb[j], acc0);
        acc1 = mfma_bf16(ra[j + 1], hb[j + 1], acc1);
      }
    }
  }
  part[wave][lane] = acc0 + acc1;
  __syncthreads();
  if (wave != 0 || !colv) return;
  const f32x4_t s = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);

  // ---- the epilogue: gates of this lane's unit(s) for batch row b; the step's states out
  const long long obase = b * a.out_sb + (long long)ts * a.out_st + (long long)n * D;
  const long long hbase = ((long long)n * a.B + b) * D;  // hbuf
  const long long lbase = b * a.last_sb + (long long)n * a.last_sn;
  const bool last = t == a.T - 1;
  auto put_h = [&](int u, float h) {
    if (rf) reinterpret_cast<float*>(hout)[hbase + u] = h;
    else reinterpret_cast<uint16_t*>(hout)[hbase + u] = f2bf(h);
    if (a.out_h) a.out_h[obase + u] = h;
    if (last && a.last_h) a.last_h[lbase + u] = h;
  };
  if (GS == 4) {
    if (a.cell == CELL_LSTM) {
      const float ig = sigmoid_f(s[0] + pin[0]), fg = sigmoid_f(s[1] + pin[1]);
      const float zg = tanh_f(s[2] + pin[2]), og = sigmoid_f(s[3] + pin[3]);
      const float c = fg * cprev + ig * zg;
      a.ccur[sbase + ue] = c;
      put_h(ue, og * tanh_f(c));
      if (a.out_c) a.out_c[obase + ue] = c;
      if (last && a.last_c) a.last_c[lbase + ue] = c;
    } else {  // GRU: the reset gate scales the candidate's recurrent part (h.R_n + b_n), not its Wx
      const float rg = sigmoid_f(s[0] + pin[0]);
      const float zg = sigmoid_f(s[1] + pin[1]);
      const float ng = tanh_f(pin[2] + rg * (s[2] + bn));
      const float h = ng + zg * (cprev - ng);  // (1 - z) n + z h
      a.ccur[sbase + ue] = h;
      put_h(ue, h);
    }
  } else {  // Elman: rows 4 quad .. +3 of the tile are four units
#pragma unroll
    for (int i = 0; i < 4; ++i) put_h(ue + i, tanh_f(s[i] + pin[i]));
  }
}

}  // namespace frnn
