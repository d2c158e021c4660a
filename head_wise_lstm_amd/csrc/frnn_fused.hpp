// Persistent fused forward recurrence for gfx950.
//
// Work split. A "group" is one head n and one block of BR <= 16 batch rows; groups never
// interact. The G*D rows of R^T of a head are cut into 16-row tiles; an LSTM tile holds the four
// gates (i, f, z, o) of four consecutive hidden units (row m = 4*unit + gate), an Elman tile
// sixteen units. W workgroups share a group, each owning MT_WG consecutive tiles; their R^T
// fragments stay in VGPRs for all T steps (the page's "weights kept in registers").
//
// Per step, each of the 4 waves of a workgroup runs MFMA v_mfma_f32_16x16x32_bf16 with
//   A = R^T tile (16 rows x 32 k), B = h^T (32 k x 16 batch columns), D = pre-activations,
// so that lane l ends up holding all four gates of unit (4*tile + l/16) for batch column l%16:
// the gate math needs no cross-lane traffic. With KS > 1 the waves split K and the partial sums
// are added through LDS.
//
// h exchange between the W workgroups of a group (W > 1): every group is placed on one
// accelerator die (XCD), whose L2 is shared by its 32 CUs. A new h value travels as a 32-bit word
// (bf16 << 16 | step tag) written with a plain store (CU caches are write-through to the die's L2)
// and is read back with 64-bit agent-scope atomic loads, which bypass the reader's CU cache. Every
// 32-bit half carries its own tag, so a reader never needs a flag, a fence or a second round trip:
// a word is either the current step's or it is polled again. Two parities of the buffer alternate
// by step. Placement is checked against the hardware XCC id; a workgroup on the wrong die reports
// an error instead of computing. Every wait is bounded by a wall-clock limit.
//
// With W == 1 ("LOCAL") the whole head sits in one workgroup and h is exchanged through LDS.
#pragma once

#include <type_traits>

#include "frnn_device.hpp"

namespace frnn {

struct FusedArgs {
  int B, T, N, D;
  int BR;       // batch rows per group (1..16)
  int groups;   // N * ceil(B / BR)
  int W;        // workgroups per group (1 for the LDS-local design)
  int n_xcd;    // dies the grid is spread over: workgroup index = slot * n_xcd + die
  int check_xcc;
  int xcc_of[8];  // expected hardware XCC id of die slot d
  const void* Wx;
  int wx_f32;
  long long wx_sb, wx_st;  // element strides of Wx for b and t; [G][N][D] packed inside
  const void* R;
  long long r_sg, r_sn, r_sd;  // element strides of R for g, n, d; e contiguous
  const void* bias;            // [G][N][D], same dtype as R, or null
  const void* s0_h;
  const void* s0_c;
  int s0_f32;
  long long s0_sb;  // element stride of the initial states for b; [N][D] packed inside
  float* out_h;
  float* out_c;
  long long out_sb, out_st;  // element strides of the state outputs for b and t
  float* last_h;
  float* last_c;
  long long last_sb;
  uint32_t* xbuf;  // exchange words [groups][2][BR][D]
  int* err;
  long long timeout_ticks;  // bound of every wait, in wall-clock (100 MHz) ticks
};

// LDS bytes the kernel needs (dynamic shared memory).
__host__ __device__ constexpr int fused_hpad(bool f32) { return f32 ? 4 : 8; }

template <int CELL, bool F32, bool LOCAL, int KS, int MTW, int KTW>
__global__ void __launch_bounds__(256, 1) fused_fwd_kernel(FusedArgs a) {
  constexpr int MS = 4 / KS;
  constexpr int MT_WG = MTW * MS;
  constexpr int KW = F32 ? 4 : 32;
  constexpr int GT = (KS == 1) ? MTW : (MT_WG + 3) / 4;
  constexpr int G = (CELL == CELL_LSTM) ? 4 : 1;
  static_assert(KS == 1 || KS == 2 || KS == 4, "KS");
  static_assert(!(F32 && !LOCAL), "fp32 runs only in the workgroup-local design");
  static_assert(!(LOCAL && KS != 1), "the workgroup-local design does not split K");
  typedef typename std::conditional<F32, float, bf16x8_t>::type frag_t;

  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int s_abort;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ks = wave % KS, ms = wave / KS;
  const int col = lane & 15, quad = lane >> 4;
  const int D = a.D, N = a.N, T = a.T;
  const int TPH = (G * D) / 16;

  int group, w;
  if (LOCAL) {
    group = blockIdx.x;
    w = 0;
  } else {
    const int die = blockIdx.x % a.n_xcd, slot = blockIdx.x / a.n_xcd;
    group = (slot / a.W) * a.n_xcd + die;
    w = slot % a.W;
    if (group >= a.groups) return;
    if (a.check_xcc && xcc_id() != a.xcc_of[die]) {
      if (threadIdx.x == 0) atomicOr(a.err, DEVERR_PLACEMENT);
      return;
    }
  }
  if (group >= a.groups) return;
  if (threadIdx.x == 0) s_abort = 0;

  const int n = group % N, bblk = group / N;
  const int b0 = bblk * a.BR;
  const int nvalid = min(a.BR, a.B - b0);
  const int tile0 = w * MT_WG;
  const bool colv = col < nvalid;
  const long long bcol = b0 + col;
  const bool r_f32 = F32;

  // ---- R^T fragments, resident for the whole sequence.
  frag_t Ra[MTW][KTW];
#pragma unroll
  for (int j = 0; j < MTW; ++j) {
    const int tt = tile0 + ms * MTW + j;
    const bool tv = tt < TPH;
    int u, g;
    if (CELL == CELL_LSTM) { u = 4 * tt + (col >> 2); g = col & 3; }
    else { u = 16 * tt + col; g = 0; }
    const long long rbase = (long long)g * a.r_sg + (long long)n * a.r_sn + u;
#pragma unroll
    for (int kk = 0; kk < KTW; ++kk) {
      if constexpr (F32) {
        const int k = (ks * KTW + kk) * KW + quad;
        Ra[j][kk] = tv ? reinterpret_cast<const float*>(a.R)[rbase + (long long)k * a.r_sd] : 0.0f;
      } else {
        const int k = (ks * KTW + kk) * KW + 8 * quad;
        const uint16_t* Rp = reinterpret_cast<const uint16_t*>(a.R);
        u32x4_t pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t lo = tv ? Rp[rbase + (long long)(k + 2 * i) * a.r_sd] : 0u;
          uint32_t hi = tv ? Rp[rbase + (long long)(k + 2 * i + 1) * a.r_sd] : 0u;
          pk[i] = lo | (hi << 16);
        }
        Ra[j][kk] = __builtin_bit_cast(bf16x8_t, pk);
      }
    }
  }

  // ---- tiles this wave applies the gates to, their bias, initial c and Wx.
  int gu[GT];       // LSTM: the lane's unit; Elman: first of the lane's four units
  bool gval[GT];
  float bia[GT][4], wxv[GT][4], creg[GT];
#pragma unroll
  for (int q = 0; q < GT; ++q) {
    const int tq = (KS == 1) ? ms * MTW + q : wave + 4 * q;
    const int tt = tile0 + tq;
    gval[q] = (tq < MT_WG) && (tt < TPH);
    gu[q] = (CELL == CELL_LSTM) ? 4 * tt + quad : 16 * tt + 4 * quad;
    creg[q] = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bia[q][i] = 0.0f;
      wxv[q][i] = 0.0f;
    }
    if (gval[q]) {
      if (a.bias) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const long long off = (CELL == CELL_LSTM) ? (long long)(i * N + n) * D + gu[q] : (long long)n * D + gu[q] + i;
          bia[q][i] = ld_f(a.bias, off, r_f32);
        }
      }
      if (CELL == CELL_LSTM && a.s0_c && colv)
        creg[q] = ld_f(a.s0_c, bcol * a.s0_sb + (long long)n * D + gu[q], a.s0_f32);
    }
  }
  auto load_wx = [&](int t) {
#pragma unroll
    for (int q = 0; q < GT; ++q) {
      if (gval[q] && colv) {
        const long long base = bcol * a.wx_sb + (long long)t * a.wx_st;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const long long off = (CELL == CELL_LSTM) ? (long long)(i * N + n) * D + gu[q] : (long long)n * D + gu[q] + i;
          wxv[q][i] = ld_f(a.Wx, base + off, a.wx_f32);
        }
      }
    }
  };

  // ---- LDS layout.
  constexpr int HPAD = fused_hpad(F32);
  const int HS = D + HPAD;  // row stride of the LDS h buffer (elements)
  float* hbuf_f = reinterpret_cast<float*>(smem);
  uint16_t* hbuf_b = reinterpret_cast<uint16_t*>(smem);
  f32x4_t* part = reinterpret_cast<f32x4_t*>(smem);

  if (LOCAL) {
    // h_{-1} (the initial state) goes to parity 1.
    for (int idx = threadIdx.x; idx < 16 * D; idx += 256) {
      const int c = idx / D, k = idx - c * D;
      float v = 0.0f;
      if (a.s0_h && c < nvalid) v = ld_f(a.s0_h, (long long)(b0 + c) * a.s0_sb + (long long)n * D + k, a.s0_f32);
      if (F32) hbuf_f[(1 * 16 + c) * HS + k] = v;
      else hbuf_b[(1 * 16 + c) * HS + k] = f2bf(v);
    }
  }
  load_wx(0);
  __syncthreads();

  const long long xgroup = (long long)group * 2 * a.BR * D;

  for (int t = 0; t < T; ++t) {
    frag_t Bf[KTW];
    // ---- 1. h_{t-1} as the B operand.
    if (LOCAL) {
      const int p = (t + 1) & 1;
#pragma unroll
      for (int kk = 0; kk < KTW; ++kk) {
        if constexpr (F32) Bf[kk] = hbuf_f[(p * 16 + col) * HS + kk * KW + quad];
        else Bf[kk] = *reinterpret_cast<const bf16x8_t*>(&hbuf_b[(p * 16 + col) * HS + kk * KW + 8 * quad]);
      }
    } else if constexpr (!F32) {
      if (t == 0) {
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk) {
          u32x4_t pk = {0u, 0u, 0u, 0u};
          if (colv && a.s0_h) {
            const long long base = bcol * a.s0_sb + (long long)n * D + (ks * KTW + kk) * 32 + 8 * quad;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              uint32_t lo = f2bf(ld_f(a.s0_h, base + 2 * i, a.s0_f32));
              uint32_t hi = f2bf(ld_f(a.s0_h, base + 2 * i + 1, a.s0_f32));
              pk[i] = lo | (hi << 16);
            }
          }
          Bf[kk] = __builtin_bit_cast(bf16x8_t, pk);
        }
      } else {
        const int pp = (t - 1) & 1;
        const uint32_t tag = (uint32_t)t & 0xFFFFu;
        const uint32_t* rowp = a.xbuf + xgroup + ((long long)pp * a.BR + col) * D + 8 * quad;
        uint32_t pend = colv ? ((1u << KTW) - 1u) : 0u;
        uint64_t v[KTW][4];
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk) Bf[kk] = __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
        long long t_first = 0;
        int spins = 0;
        bool dead = false;
        while (true) {
#pragma unroll
          for (int kk = 0; kk < KTW; ++kk) {
            if (pend & (1u << kk)) {
              const uint64_t* src = reinterpret_cast<const uint64_t*>(rowp + (ks * KTW + kk) * 32);
#pragma unroll
              for (int i = 0; i < 4; ++i)
                v[kk][i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
#pragma unroll
          for (int kk = 0; kk < KTW; ++kk) {
            if (pend & (1u << kk)) {
              uint32_t bad = 0;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const uint32_t lo = (uint32_t)v[kk][i], hi = (uint32_t)(v[kk][i] >> 32);
                bad |= ((lo ^ tag) | (hi ^ tag)) & 0xFFFFu;
              }
              if (bad == 0) {
                u32x4_t pk;
#pragma unroll
                for (int i = 0; i < 4; ++i) pk[i] = pack_hi((uint32_t)v[kk][i], (uint32_t)(v[kk][i] >> 32));
                Bf[kk] = __builtin_bit_cast(bf16x8_t, pk);
                pend &= ~(1u << kk);
              }
            }
          }
          if (!__any(pend != 0u)) break;
          if ((++spins & 63) == 0) {
            const long long now = (long long)wall_clock64();
            if (t_first == 0) t_first = now;
            if (now - t_first > a.timeout_ticks ||
                __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
              if (lane == 0) atomicOr(a.err, DEVERR_TIMEOUT);
              dead = true;
              break;
            }
          }
        }
        if (dead) {
          if (KS == 1) return;  // no workgroup barrier in this loop: leave directly
          s_abort = 1;
        }
      }
    }

    // ---- 2. recurrent contraction on MFMA.
    f32x4_t acc[MTW];
#pragma unroll
    for (int j = 0; j < MTW; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KTW; ++kk) {
#pragma unroll
      for (int j = 0; j < MTW; ++j) {
        if constexpr (F32) acc[j] = mfma_f32(Ra[j][kk], Bf[kk], acc[j]);
        else acc[j] = mfma_bf16(Ra[j][kk], Bf[kk], acc[j]);
      }
    }

    // ---- 3. K-split partial sums through LDS.
    f32x4_t pre[GT];
    if constexpr (KS == 1) {
#pragma unroll
      for (int q = 0; q < GT; ++q) pre[q] = acc[q];
    } else {
      const int pp = t & 1;
#pragma unroll
      for (int j = 0; j < MTW; ++j) part[((pp * KS + ks) * MT_WG + ms * MTW + j) * 64 + lane] = acc[j];
      __syncthreads();
      if (s_abort) return;
#pragma unroll
      for (int q = 0; q < GT; ++q) {
        pre[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (gval[q]) {
          const int tq = wave + 4 * q;
#pragma unroll
          for (int k2 = 0; k2 < KS; ++k2) pre[q] += part[((pp * KS + k2) * MT_WG + tq) * 64 + lane];
        }
      }
    }

    // ---- 4. gates, state update, outputs, exchange.
    const uint32_t wtag = (uint32_t)(t + 1) & 0xFFFFu;
#pragma unroll
    for (int q = 0; q < GT; ++q) {
      if (!gval[q]) continue;
      if constexpr (CELL == CELL_LSTM) {
        const float ig = sigmoid_f(pre[q][0] + wxv[q][0] + bia[q][0]);
        const float fg = sigmoid_f(pre[q][1] + wxv[q][1] + bia[q][1]);
        const float zg = tanh_f(pre[q][2] + wxv[q][2] + bia[q][2]);
        const float og = sigmoid_f(pre[q][3] + wxv[q][3] + bia[q][3]);
        const float c = fg * creg[q] + ig * zg;
        creg[q] = c;
        const float h = og * tanh_f(c);
        const int u = gu[q];
        if (colv) {
          const long long o = bcol * a.out_sb + (long long)t * a.out_st + (long long)n * D + u;
          if (a.out_h) a.out_h[o] = h;
          if (a.out_c) a.out_c[o] = c;
          if (t == T - 1) {
            const long long lo = bcol * a.last_sb + (long long)n * D + u;
            if (a.last_h) a.last_h[lo] = h;
            if (a.last_c) a.last_c[lo] = c;
          }
        }
        if (LOCAL) {
          if constexpr (F32) hbuf_f[((t & 1) * 16 + col) * HS + u] = h;
          else hbuf_b[((t & 1) * 16 + col) * HS + u] = f2bf(h);
        } else if (colv) {
          a.xbuf[xgroup + ((long long)(t & 1) * a.BR + col) * D + u] = ((uint32_t)f2bf(h) << 16) | wtag;
        }
      } else {
        float h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = tanh_f(pre[q][i] + wxv[q][i] + bia[q][i]);
        const int u = gu[q];
        if (colv) {
          const long long o = bcol * a.out_sb + (long long)t * a.out_st + (long long)n * D + u;
          if (a.out_h) *reinterpret_cast<f32x4_t*>(a.out_h + o) = f32x4_t{h[0], h[1], h[2], h[3]};
          if (t == T - 1 && a.last_h)
            *reinterpret_cast<f32x4_t*>(a.last_h + bcol * a.last_sb + (long long)n * D + u) = f32x4_t{h[0], h[1], h[2], h[3]};
        }
        if (LOCAL) {
          if constexpr (F32) {
            *reinterpret_cast<f32x4_t*>(&hbuf_f[((t & 1) * 16 + col) * HS + u]) = f32x4_t{h[0], h[1], h[2], h[3]};
          } else {
            u16x4_t hv = {f2bf(h[0]), f2bf(h[1]), f2bf(h[2]), f2bf(h[3])};
            *reinterpret_cast<u16x4_t*>(&hbuf_b[((t & 1) * 16 + col) * HS + u]) = hv;
          }
        } else if (colv) {
          u32x4_t wv;
#pragma unroll
          for (int i = 0; i < 4; ++i) wv[i] = ((uint32_t)f2bf(h[i]) << 16) | wtag;
          *reinterpret_cast<u32x4_t*>(a.xbuf + xgroup + ((long long)(t & 1) * a.BR + col) * D + u) = wv;
        }
      }
    }
    // Keep the exchange stores ahead of the next step's polling in program order.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (t + 1 < T) load_wx(t + 1);
    if (LOCAL) __syncthreads();
  }
}

}  // namespace frnn
