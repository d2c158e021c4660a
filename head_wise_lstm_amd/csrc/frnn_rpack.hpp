// R^T in MFMA A-fragment order, shared by both recurrence paths.
//
// The recurrent contraction of a head is pre[g][e] = sum_d h[d] R[g][n][d][e] (h as a row vector
// times R, the reading the pages' single-layer form matmul(h, Wh) fixes). On MFMA the rows of the
// A operand are the outputs: a 16-row tile of R^T holds the four gate rows of four consecutive
// hidden units (row m = 4*unit + gate; a GRU unit's fourth row is zero; an Elman tile holds
// sixteen units), and one k-tile is 32 values of d
// (bf16, v_mfma_f32_16x16x32_bf16) or 4 (fp32, v_mfma_f32_16x16x4f32). Lane l = 16*quad + m of a
// fragment holds row m at k = 8*quad .. 8*quad+7 (bf16) or k = quad (fp32).
//
// Packed layout: [N][TPH][KT][64 lanes] x (8 bf16 | 1 fp32), TPH = slots*D/16 tiles (slots = 4
// rows per unit, or 1 for Elman), KT = D/32 (bf16) or D/4 (fp32) k-tiles; it has slots*N*D*D
// elements (as many as R, a third more for the GRU).
#pragma once

#include "frnn_device.hpp"

namespace frnn {

struct RpackArgs {
  int N, D, cell;
  const void* R;
  long long r_sg, r_sn, r_sd;  // element strides of R for g, n, d; e contiguous
  void* out;
};

constexpr int RPACK_UB = 64;  // hidden units per block of the bf16 pack kernel

// bf16: one block per (64-unit block, k-tile, head). R rows (g, d) are read 8 bytes per thread,
// 16 threads per 128-byte row (coalesced), into LDS; the fragments are then gathered from LDS and
// written 16 bytes per lane. Needs e-stride 1 and g/n/d strides that are multiples of 4 elements.
__global__ void __launch_bounds__(256) rpack_bf16_kernel(RpackArgs a) {
  constexpr int SROW = RPACK_UB + 8;  // LDS row stride (elements)
  __shared__ uint16_t s[4 * 32 * SROW];
  const int G = cell_gates(a.cell), GS = cell_slots(a.cell);
  const int UPT = GS == 4 ? 4 : 16;
  const int TPH = GS * a.D / 16, KT = a.D / 32;
  const int ub = blockIdx.x, kt = blockIdx.y, n = blockIdx.z;
  const int u0 = ub * RPACK_UB;
  const uint16_t* R = reinterpret_cast<const uint16_t*>(a.R);
  // stage: rows r = g*32 + dd, units u0 .. u0+63
  for (int i = threadIdx.x; i < G * 32 * (RPACK_UB / 4); i += 256) {
    const int r = i / (RPACK_UB / 4), c4 = (i % (RPACK_UB / 4)) * 4;
    const int g = r / 32, dd = r % 32;
    uint2 v = make_uint2(0u, 0u);
    if (u0 + c4 < a.D)
      v = *reinterpret_cast<const uint2*>(R + (long long)g * a.r_sg + (long long)n * a.r_sn +
                                          (long long)(kt * 32 + dd) * a.r_sd + u0 + c4);
    *reinterpret_cast<uint2*>(&s[r * SROW + c4]) = v;
  }
  __syncthreads();
  const int tiles = RPACK_UB / UPT;
  for (int i = threadIdx.x; i < tiles * 64; i += 256) {
    const int tl = i / 64, lane = i % 64;
    const int tt = ub * tiles + tl;
    if (tt >= TPH) continue;
    const int m = lane & 15, quad = lane >> 4;
    int ul, g;
    if (GS == 4) { ul = 4 * tl + (m >> 2); g = m & 3; }
    else { ul = 16 * tl + m; g = 0; }
    u32x4_t pk = {0u, 0u, 0u, 0u};  // rows of gates the cell does not have stay zero
    if (g < G) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = s[(g * 32 + 8 * quad + 2 * j) * SROW + ul];
        const uint32_t hi = s[(g * 32 + 8 * quad + 2 * j + 1) * SROW + ul];
        pk[j] = lo | (hi << 16);
      }
    }
    reinterpret_cast<u32x4_t*>(a.out)[(((long long)n * TPH + tt) * KT + kt) * 64 + lane] = pk;
  }
}

// Any strides and fp32: one thread per (head, tile, k-tile, lane) gathers its values directly.
__global__ void __launch_bounds__(256) rpack_any_kernel(RpackArgs a, int f32) {
  const int G = cell_gates(a.cell), GS = cell_slots(a.cell);
  const int TPH = GS * a.D / 16;
  const int KT = a.D / (f32 ? 4 : 32);
  const long long total = (long long)a.N * TPH * KT * 64;
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (long long)gridDim.x * 256) {
    const int lane = (int)(idx & 63);
    long long r = idx >> 6;
    const int kt = (int)(r % KT);
    r /= KT;
    const int tt = (int)(r % TPH);
    const int n = (int)(r / TPH);
    const int m = lane & 15, quad = lane >> 4;
    int u, g;
    if (GS == 4) { u = 4 * tt + (m >> 2); g = m & 3; }
    else { u = 16 * tt + m; g = 0; }
    const bool gv = g < G;  // rows of gates the cell does not have are zero
    const long long base = (long long)(gv ? g : 0) * a.r_sg + (long long)n * a.r_sn + u;
    if (f32) {
      reinterpret_cast<float*>(a.out)[idx] =
          gv ? reinterpret_cast<const float*>(a.R)[base + (long long)(kt * 4 + quad) * a.r_sd] : 0.0f;
    } else {
      const uint16_t* Rp = reinterpret_cast<const uint16_t*>(a.R);
      const int k = kt * 32 + 8 * quad;
      u32x4_t pk = {0u, 0u, 0u, 0u};
      if (gv) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pk[i] = (uint32_t)Rp[base + (long long)(k + 2 * i) * a.r_sd] |
                  ((uint32_t)Rp[base + (long long)(k + 2 * i + 1) * a.r_sd] << 16);
      }
      reinterpret_cast<u32x4_t*>(a.out)[idx] = pk;
    }
  }
}

}  // namespace frnn
