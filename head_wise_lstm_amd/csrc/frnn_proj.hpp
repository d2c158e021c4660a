// Input projection of the multi-layer LSTM ("5.3 LSTM": x_t . Wi + bias_ih + bias_hh) for all T
// steps at once, as one MFMA GEMM:  C[M][Nc] (fp32) = A[M][K] . Wi[K][Nc] + b1[Nc] + b2[Nc].
// A is bf16 or fp32 (rounded to bf16 as it is staged), Wi and the biases bf16, row-major.
//
// Wi is first transposed to Bt[Nc][K] (transpose_kernel), so that both operands are read
// as rows of K: every global load is 16 contiguous bytes and every MFMA fragment one 16-byte LDS
// read. The GEMM runs 256 x 128 output tiles per workgroup; each of the 4 waves owns 128 x 64
// (8 x 4 tiles of v_mfma_f32_16x16x32_bf16, 32 accumulators), which keeps LDS traffic at about
// 96 bytes per clock per CU. K goes 32 at a time through two LDS buffers: the next step's global
// loads are in flight in registers while the current step's MFMAs run, one barrier per step.
// With bf16 A, proj_gemm_dma_kernel loads the same tiles straight into a three-stage LDS ring.
#pragma once

#include <type_traits>

#include "frnn_device.hpp"

namespace frnn {

struct ProjArgs {
  int M, Nc, K;      // K a multiple of 32
  const void* A;
  int a_f32;
  long long lda;
  const uint16_t* Bt;  // [Nc][K] bf16 (Wi transposed), rows ldb apart
  long long ldb;
  const uint16_t* b1;
  const uint16_t* b2;
  float* C;
  long long ldc;
  long long a_z, b_z, c_z;  // element offsets of A, Bt and C per blockIdx.y (independent parts)
  long long a_h, b_h, c_h;  // and per blockIdx.z (heads; a second batch dimension)
  int nt;  // 1: C by streaming stores (read later by a streaming kernel, not by a recurrence)
};

// (a compile-time choice: with a run-time one the compiler merges both stores into the plain one)
template <bool NT>
__device__ __forceinline__ void proj_put(float* c, float v) {
  if constexpr (NT) __builtin_nontemporal_store(v, c);
  else *c = v;
}

constexpr int PJ_BM = 256, PJ_BN = 128, PJ_BK = 32;
constexpr int PJ_DIES = 8;  // accelerator dies (XCDs) of an MI355X
constexpr int PJ_LS = PJ_BK + 8;  // LDS row stride (bf16): 80 bytes, spreads a fragment's rows over the banks

// dst[j][k] = src[k][j] for k < K, j < Nc (src row stride lds, dst row stride ldd), 32 x 32 tiles
// through LDS. Grid (ceil(Nc/32), min(ceil(K/32), 65535), matrices); the y tiles repeat by
// gridDim.y; matrix z starts src_z and dst_z elements further.
template <typename E>
__global__ void __launch_bounds__(256) transpose_kernel(const E* src, long long lds, int K, int Nc, E* dst,
                                                        long long ldd, long long src_z, long long dst_z) {
  __shared__ E s[32][33];
  src += blockIdx.z * src_z;
  dst += blockIdx.z * dst_z;
  const int n0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int kb = blockIdx.y; kb * 32 < K; kb += gridDim.y) {
    const int k0 = kb * 32;
#pragma unroll
    for (int i = 0; i < 32; i += 8) {
      const int k = k0 + ty + i, n = n0 + tx;
      s[ty + i][tx] = (k < K && n < Nc) ? src[(long long)k * lds + n] : (E)0;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 32; i += 8) {
      const int n = n0 + ty + i, k = k0 + tx;
      if (n < Nc && k < K) dst[(long long)n * ldd + k] = s[tx][ty + i];
    }
    __syncthreads();
  }
}

// dst[j][k] = src[k][j] for 16-bit elements on 64 x 64 tiles: every global access is 4
// consecutive elements (8 bytes) of a row, so a wave moves 512 contiguous-in-rows bytes per
// instruction instead of 128. Needs src, dst 8-byte aligned and lds, ldd multiples of 4; tiles
// that cross the K or Nc edge move element by element. Grid (ceil(Nc/64), min(ceil(K/64), 65535),
// matrices), matrix z starting src_z and dst_z elements further (multiples of 4).
__global__ void __launch_bounds__(256) transpose_b16_kernel(const uint16_t* src, long long lds, int K, int Nc,
                                                            uint16_t* dst, long long ldd, long long src_z,
                                                            long long dst_z) {
  __shared__ __attribute__((aligned(16))) uint16_t s[64][68];
  src += blockIdx.z * src_z;
  dst += blockIdx.z * dst_z;
  const int n0 = blockIdx.x * 64;
  const int t = threadIdx.x, r = t >> 4, c4 = (t & 15) * 4;  // row r + 16 i, 4 elements from c4
  for (int kb = blockIdx.y; kb * 64 < K; kb += gridDim.y) {
    const int k0 = kb * 64;
    const bool full = k0 + 64 <= K && n0 + 64 <= Nc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = k0 + r + 16 * i;
      uint2 v;
      if (full) {
        v = *reinterpret_cast<const uint2*>(src + (long long)k * lds + n0 + c4);
      } else {
        uint16_t e[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + c4 + q;
          e[q] = (k < K && n < Nc) ? src[(long long)k * lds + n] : (uint16_t)0;
        }
        v.x = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
        v.y = (uint32_t)e[2] | ((uint32_t)e[3] << 16);
      }
      *reinterpret_cast<uint2*>(&s[r + 16 * i][c4]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = r + 16 * i;  // output row (input column n0 + j), 4 elements from k0 + c4
      uint2 v;
      v.x = (uint32_t)s[c4][j] | ((uint32_t)s[c4 + 1][j] << 16);
      v.y = (uint32_t)s[c4 + 2][j] | ((uint32_t)s[c4 + 3][j] << 16);
      const int n = n0 + j;
      if (full) {
        *reinterpret_cast<uint2*>(dst + (long long)n * ldd + k0 + c4) = v;
      } else if (n < Nc) {
        const uint16_t e[4] = {(uint16_t)(v.x & 0xFFFFu), (uint16_t)(v.x >> 16), (uint16_t)(v.y & 0xFFFFu),
                               (uint16_t)(v.y >> 16)};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (k0 + c4 + q < K) dst[(long long)n * ldd + k0 + c4 + q] = e[q];
      }
    }
    __syncthreads();
  }
}

// dst[j][k] = bf16(src[k][j]) for fp32 src (as transpose_kernel, rounding to nearest even).
__global__ void __launch_bounds__(256) transpose_f32_bf16_kernel(const float* src, long long lds, int K, int Nc,
                                                                 uint16_t* dst, long long ldd) {
  __shared__ float s[32][33];
  const int n0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int kb = blockIdx.y; kb * 32 < K; kb += gridDim.y) {
    const int k0 = kb * 32;
#pragma unroll
    for (int i = 0; i < 32; i += 8) {
      const int k = k0 + ty + i, n = n0 + tx;
      s[ty + i][tx] = (k < K && n < Nc) ? src[(long long)k * lds + n] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 32; i += 8) {
      const int n = n0 + ty + i, k = k0 + tx;
      if (n < Nc && k < K) dst[(long long)n * ldd + k] = f2bf(s[tx][ty + i]);
    }
    __syncthreads();
  }
}

// out[i] = sum over p < parts of in[p * n + i], in order (the K parts of a split GEMM).
__global__ void __launch_bounds__(256) sum_parts_kernel(const float* in, int parts, long long n, float* out) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    float v = 0.0f;
    for (int p = 0; p < parts; ++p) v += in[p * n + i];
    out[i] = v;
  }
}

// Staging of 8 consecutive k of one row in registers: 16 bytes of bf16, or 32 bytes of fp32 kept
// raw (rounded to bf16 only when written to LDS, so that no load is waited for when issued).
template <bool F32>
struct Stage8 {
  typename std::conditional<F32, f32x4_t, u32x4_t>::type v[F32 ? 2 : 1];
};

template <bool F32>
__device__ __forceinline__ void proj_load8(Stage8<F32>& st, const void* base, long long ld, long long r, long long rows,
                                           int k) {
  const bool ok = r < rows;
  const long long rr = ok ? r : 0;  // rows past the end load row 0 and are zeroed when stored
  if constexpr (F32) {
    const float* p = reinterpret_cast<const float*>(base) + rr * ld + k;
    st.v[0] = *reinterpret_cast<const f32x4_t*>(p);
    st.v[1] = *reinterpret_cast<const f32x4_t*>(p + 4);
    if (!ok) st.v[0] = st.v[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  } else {
    st.v[0] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(base) + rr * ld + k);
    if (!ok) st.v[0] = u32x4_t{0u, 0u, 0u, 0u};
  }
}

template <bool F32>
__device__ __forceinline__ void proj_store8(uint16_t* dst, const Stage8<F32>& st) {
  u32x4_t v;
  if constexpr (F32) {
    v[0] = (uint32_t)f2bf(st.v[0][0]) | ((uint32_t)f2bf(st.v[0][1]) << 16);
    v[1] = (uint32_t)f2bf(st.v[0][2]) | ((uint32_t)f2bf(st.v[0][3]) << 16);
    v[2] = (uint32_t)f2bf(st.v[1][0]) | ((uint32_t)f2bf(st.v[1][1]) << 16);
    v[3] = (uint32_t)f2bf(st.v[1][2]) | ((uint32_t)f2bf(st.v[1][3]) << 16);
  } else {
    v = st.v[0];
  }
  *reinterpret_cast<u32x4_t*>(dst) = v;
}

// AF32: A is fp32. Two workgroups per CU: while one waits for its loads, the other multiplies.
template <bool AF32, bool NT>
__global__ void __launch_bounds__(256, 2) proj_gemm_kernel(ProjArgs p) {
  // two stages of A (256 x 32) and B (128 x 32), rows padded to PJ_LS
  __shared__ __attribute__((aligned(16))) uint16_t As[2][PJ_BM * PJ_LS];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][PJ_BN * PJ_LS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, quad = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;  // wave tile: rows wm*128 .., columns wn*64 ..
  if (blockIdx.y || blockIdx.z) {  // part y of head z of a batch of independent products
    p.A = reinterpret_cast<const char*>(p.A) + (blockIdx.y * p.a_z + blockIdx.z * p.a_h) * (AF32 ? 4 : 2);
    p.Bt += blockIdx.y * p.b_z + blockIdx.z * p.b_h;
    p.C += blockIdx.y * p.c_z + blockIdx.z * p.c_h;
  }
  // Die-aware tile order. Workgroups are dealt to the 8 dies round-robin by index, so the die of
  // workgroup L is L % 8. Tiles are numbered row-major (M tile, then N tile) and each die takes a
  // contiguous run of them: the N tiles that share an A tile run on one die and read A once into
  // its L2 (dealt in index order, the A tile would be read by every die).
  const int ntn = (p.Nc + PJ_BN - 1) / PJ_BN;
  const int L = blockIdx.x, G = gridDim.x;
  const int tile = (G % PJ_DIES == 0) ? (L % PJ_DIES) * (G / PJ_DIES) + L / PJ_DIES : L;
  const long long m0 = (long long)(tile / ntn) * PJ_BM;
  const int n0 = (tile % ntn) * PJ_BN;

  // global -> register staging of the next K step: A 256 rows x 4 chunks of 8 k (4 per thread),
  // B 128 x 4 (2 per thread); chunk c of thread tid is row tid / 4 + 64 c, k-chunk tid % 4
  Stage8<AF32> ra[4];
  Stage8<false> rb[2];
  const int lrow = tid >> 2, lkc = (tid & 3) * 8;
  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = p.K / PJ_BK;
#define PJ_GLOAD(K0)                                                                              \
  do {                                                                                            \
    _Pragma("unroll") for (int c = 0; c < 4; ++c)                                                 \
      proj_load8<AF32>(ra[c], p.A, p.lda, m0 + lrow + 64 * c, p.M, (K0) + lkc);                   \
    _Pragma("unroll") for (int c = 0; c < 2; ++c)                                                 \
      proj_load8<false>(rb[c], p.Bt, p.ldb, (long long)n0 + lrow + 64 * c, p.Nc, (K0) + lkc);     \
  } while (0)
#define PJ_LSTORE(ST)                                                                             \
  do {                                                                                            \
    _Pragma("unroll") for (int c = 0; c < 4; ++c)                                                 \
      proj_store8<AF32>(&As[ST][(lrow + 64 * c) * PJ_LS + lkc], ra[c]);                           \
    _Pragma("unroll") for (int c = 0; c < 2; ++c)                                                 \
      proj_store8<false>(&Bs[ST][(lrow + 64 * c) * PJ_LS + lkc], rb[c]);                          \
  } while (0)
  PJ_GLOAD(0);
  PJ_LSTORE(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) PJ_GLOAD((kt + 1) * PJ_BK);
    bf16x8_t bfr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[st][(wn * 64 + j * 16 + col) * PJ_LS + 8 * quad]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(&As[st][(wm * 128 + i * 16 + col) * PJ_LS + 8 * quad]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(af, bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) PJ_LSTORE(st ^ 1);
    __syncthreads();
  }
#undef PJ_GLOAD
#undef PJ_LSTORE
  // Epilogue: lane (col, quad) holds rows 4*quad + r of column col of every 16 x 16 tile.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int gn = n0 + wn * 64 + j * 16 + col;
    if (gn >= p.Nc) continue;
    const float bias = (p.b1 ? bf2f(p.b1[gn]) : 0.0f) + (p.b2 ? bf2f(p.b2[gn]) : 0.0f);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const long long gm = m0 + wm * 128 + i * 16 + 4 * quad + r;
        if (gm < p.M) proj_put<NT>(&p.C[gm * p.ldc + gn], acc[i][j][r] + bias);
      }
    }
  }
}

// bf16 A only: the same tiles and wave layout, with the operands loaded straight from memory into
// a ring of PD_STAGES LDS stages (16-byte global_load_lds), so that two K steps are in flight
// without staging registers. One load instruction of a wave fills 1 KB of LDS, lane l at byte
// 16 l: 16 rows of 64 bytes (32 k). Lane l therefore fetches row l / 4 of its 16-row block and the
// 16-byte chunk that belongs at position l % 4, where chunk c of row r sits at position
// c ^ ((r / 4) % 4): the 16 rows that a fragment read touches at one chunk then fall on 16
// different 16-byte bank groups. Rows past the end load the last row: only outputs that are never
// stored depend on them. A and Bt rows must start on 16-byte boundaries.
constexpr int PD_STAGES = 3;
// BM rows a tile: 256, or 128 for products of at most 128 rows (a head's dR and db, D + 1 rows),
// which would leave most of a 256-row tile's loads and MFMAs on rows past the end
__host__ __device__ constexpr int pd_a_bytes(int BM) { return BM * PJ_BK * 2; }
constexpr int PD_B_BYTES = PJ_BN * PJ_BK * 2;
__host__ __device__ constexpr int pd_stage_bytes(int BM) { return pd_a_bytes(BM) + PD_B_BYTES; }  // 24 KB at 256 rows
__host__ __device__ constexpr int pd_a_loads(int BM) { return BM / 16 / 4; }  // per wave and stage: 4 (256 rows)
constexpr int PD_B_LOADS = PJ_BN / 16 / 4;                                    // 2

typedef __attribute__((address_space(3))) void pd_lds_t;
typedef __attribute__((address_space(1))) void pd_glb_t;

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector-memory operations and no
// LDS operation remain (expcnt left alone).
__host__ __device__ constexpr int pd_vmcnt(int n) { return (n & 0xF) | (7 << 4) | ((n >> 4) << 14); }

template <bool NT, int BM = PJ_BM>
__global__ void __launch_bounds__(256, 2) proj_gemm_dma_kernel(ProjArgs p) {
  constexpr int PD_A_BYTES = pd_a_bytes(BM), PD_STAGE_BYTES = pd_stage_bytes(BM);
  constexpr int PD_A_LOADS = pd_a_loads(BM), PD_LOADS = PD_A_LOADS + PD_B_LOADS;
  constexpr int WMB = BM / 32;  // 16-row blocks of a wave's half of the tile
  __shared__ __attribute__((aligned(1024))) char ring[PD_STAGES * PD_STAGE_BYTES];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, quad = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  if (blockIdx.y || blockIdx.z) {
    p.A = reinterpret_cast<const char*>(p.A) + (blockIdx.y * p.a_z + blockIdx.z * p.a_h) * 2;
    p.Bt += blockIdx.y * p.b_z + blockIdx.z * p.b_h;
    p.C += blockIdx.y * p.c_z + blockIdx.z * p.c_h;
  }
  const int ntn = (p.Nc + PJ_BN - 1) / PJ_BN;
  const int L = blockIdx.x, G = gridDim.x;
  const int tile = (G % PJ_DIES == 0) ? (L % PJ_DIES) * (G / PJ_DIES) + L / PJ_DIES : L;
  const long long m0 = (long long)(tile / ntn) * BM;
  const int n0 = (tile % ntn) * PJ_BN;

  // this lane's source rows: A blocks PD_A_LOADS wave + e, B blocks 2 wave + e; the chunk for
  // position lane % 4
  const int brow = lane >> 2, chunk = (lane & 3) ^ ((lane >> 4) & 3);
  const char* asrc[PD_A_LOADS];
  const char* bsrc[PD_B_LOADS];
#pragma unroll
  for (int e = 0; e < PD_A_LOADS; ++e) {
    const long long r0 = m0 + 16 * (PD_A_LOADS * wave + e) + brow, r = r0 < p.M ? r0 : p.M - 1;
    asrc[e] = reinterpret_cast<const char*>(p.A) + (r * p.lda + 8 * chunk) * 2;
  }
#pragma unroll
  for (int e = 0; e < PD_B_LOADS; ++e) {
    const long long r0 = (long long)n0 + 16 * (PD_B_LOADS * wave + e) + brow, r = r0 < p.Nc ? r0 : p.Nc - 1;
    bsrc[e] = reinterpret_cast<const char*>(p.Bt + r * p.ldb + 8 * chunk);
  }
  auto issue = [&](int kt) {
    char* st = ring + (kt % PD_STAGES) * PD_STAGE_BYTES;
    const int kb = kt * PJ_BK * 2;
#pragma unroll
    for (int e = 0; e < PD_A_LOADS; ++e)
      __builtin_amdgcn_global_load_lds((pd_glb_t*)(asrc[e] + kb), (pd_lds_t*)(st + 1024 * (PD_A_LOADS * wave + e)), 16,
                                       0, 0);
#pragma unroll
    for (int e = 0; e < PD_B_LOADS; ++e)
      __builtin_amdgcn_global_load_lds((pd_glb_t*)(bsrc[e] + kb),
                                       (pd_lds_t*)(st + PD_A_BYTES + 1024 * (PD_B_LOADS * wave + e)), 16, 0, 0);
  };
  // fragment (row col of a 16-row block, k 8 quad .. 8 quad + 7)
  const int foff = col * 64 + ((quad ^ (col >> 2)) & 3) * 16;

  f32x4_t acc[WMB][4];
#pragma unroll
  for (int i = 0; i < WMB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = p.K / PJ_BK;
  if (nk > 0) issue(0);
  if (nk > 1) issue(1);
  for (int kt = 0; kt < nk; ++kt) {
    // wait for this wave's loads of step kt and its reads of step kt - 1, then for every wave's:
    // after the barrier step kt's stage is complete and step kt - 1's slot is free for step kt + 2
    asm volatile("" ::: "memory");
    if (kt + 1 < nk) __builtin_amdgcn_s_waitcnt(pd_vmcnt(PD_LOADS));
    else __builtin_amdgcn_s_waitcnt(pd_vmcnt(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + 2 < nk) issue(kt + 2);
    const char* st = ring + (kt % PD_STAGES) * PD_STAGE_BYTES;
    bf16x8_t bfr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8_t*>(st + PD_A_BYTES + 1024 * (wn * 4 + j) + foff);
#pragma unroll
    for (int i = 0; i < WMB; ++i) {
      const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(st + 1024 * (wm * WMB + i) + foff);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(af, bfr[j], acc[i][j]);
    }
  }
  // epilogue as in proj_gemm_kernel
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int gn = n0 + wn * 64 + j * 16 + col;
    if (gn >= p.Nc) continue;
    const float bias = (p.b1 ? bf2f(p.b1[gn]) : 0.0f) + (p.b2 ? bf2f(p.b2[gn]) : 0.0f);
#pragma unroll
    for (int i = 0; i < WMB; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const long long gm = m0 + wm * (BM / 2) + i * 16 + 4 * quad + r;
        if (gm < p.M) proj_put<NT>(&p.C[gm * p.ldc + gn], acc[i][j][r] + bias);
      }
    }
  }
}

}  // namespace frnn
