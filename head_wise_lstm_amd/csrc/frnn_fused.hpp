// Persistent fused forward recurrence for gfx950.
//
// Work split. A "group" is one head n and one block of BR <= 16 batch rows; groups never
// interact. The rows of R^T of a head are cut into 16-row tiles; an LSTM tile holds the four
// gates (i, f, z, o) of four consecutive hidden units (row m = 4*unit + gate), a GRU tile the
// gates r, z, n of four units in the same places (row 4*unit + 3 is zero), an Elman tile sixteen
// units. W workgroups share a group, each owning MT_WG consecutive tiles; their R^T
// fragments stay in VGPRs for all T steps (the page's "weights kept in registers").
//
// Waves. Four to eight compute waves run MFMA v_mfma_f32_16x16x32_bf16 with
//   A = R^T tile (16 rows x 32 k), B = h^T (32 k x 16 batch columns), D = pre-activations,
// so that lane l ends up holding all four gates of unit (4*tile + l/16) for batch column l%16:
// the gate math needs no cross-lane traffic. With KS > 1 the compute waves split K and add the
// partial sums through LDS. One more wave does the other global-memory traffic: it streams Wx
// several steps ahead into an LDS ring and, in the die-local design, writes the state outputs
// from an LDS ring two steps behind (in the single-workgroup design the compute waves, which
// never wait on a global load there, store the states themselves). On gfx9 a wave's vector-memory counter retires in issue order, so keeping those
// long-latency accesses out of the compute waves keeps them off the serial chain: a compute wave
// only ever waits on its own exchange traffic. One workgroup barrier per step orders the rings.
//
// h exchange between the W workgroups of a group (W > 1): every group is placed on one
// accelerator die (XCD), whose L2 is shared by its 32 CUs. A new h value travels as a 32-bit word
// (bf16 << 16 | step tag) written with a plain store (CU caches are write-through to the die's L2)
// and is read back with 8- or 16-byte loads that bypass the reader's CU cache (cache policy sc1,
// the coherence of an agent-scope atomic load). Every 32-bit word carries its own tag, so a reader
// needs no flag, fence or second round trip: a word is either the current step's or it is polled
// again, and a wide load that sees words of two steps is just polled again. Two parities of the buffer alternate by
// step. Placement is checked against the hardware XCC id; a workgroup on the wrong die reports an
// error instead of computing. Every wait is bounded by a wall-clock limit.
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
  int n_xcd;    // dies the grid is spread over (die-local design: slots workgroups on each)
  int slots;
  uint32_t xcc_of;  // hardware XCC id of die d in bits [4d, 4d+4)
  uint32_t* ctr;    // per-die workgroup counters (filled with 0xFFFF before the launch)
  const void* Wx;
  int wx_f32;
  long long wx_sb, wx_st;  // element strides of Wx for b and t; [G][N][D] packed inside
  const void* R;
  long long r_sg, r_sn, r_sd;  // element strides of R for g, n, d; e contiguous
  const void* rpack;           // bf16: R^T in fragment order [N][TPH][D/32][64] x 8 bf16
  const void* bias;            // [G][N][D], same dtype as R, or null
  const void* s0_h;
  const void* s0_c;
  int s0_f32;
  long long s0_sb, s0_sn;  // element strides of the initial states for b and n; units dense
  float* out_h;
  float* out_c;
  long long out_sb, out_st;  // element strides of the state outputs for b and t
  float* last_h;
  float* last_c;
  long long last_sb, last_sn;
  int rev_n0;  // heads n >= rev_n0 run backwards in time: step t reads Wx and writes states at T-1-t
  uint32_t* xbuf;  // exchange words [groups][2][BR][D]
  int* err;
  long long timeout_ticks;  // bound of every wait, in wall-clock (100 MHz) ticks
  int stall_step;           // a failure-handling test's hook: this step publishes a stale tag (-1: none)
};

constexpr int FUSED_IO_STAGES = 4;   // record steps in flight in the backward's I/O wave
// max 64-bit Wx words (and, in the die-local design, output pairs) one I/O lane moves per step:
// the die-local design moves few (its workgroups own few units: two words, four where a workgroup
// owns eight or more tiles, so that four batch rows of fp32 Wx fit), the single-workgroup design a
// whole head's rows of Wx (an Elman head has a quarter of an LSTM head's). Every slot costs a load
// per step.
__host__ __device__ constexpr int fused_epl(bool local, int ncw, int cell, int ks, int mtw) {
  return !local ? ((ncw / ks) * mtw >= 8 ? 4 : 2) : (cell == CELL_ELMAN ? 2 : (ncw == 4 ? 8 : 4));
}

// Wx steps in flight in the forward's I/O wave: eight where a lane moves at most two words a step
// (measured against four: Elman B=64 N=12 D=64 0.432 -> 0.394 us per step, LSTM B=16 D=768
// 1.223 -> 1.200), four where it moves more (eight stages of those spill registers).
// (A whole bf16 Elman head per workgroup streams Wx through its own LDS ring instead, see
// FUSED_DMA_STAGES; the register ring of sixteen steps measured 0.317 -> 0.305 us per step there
// against eight, and remains for fp32 Elman heads.)
__host__ __device__ constexpr int fused_io_stages(bool local, int ncw, int cell, int ks, int mtw) {
  return (local && cell == CELL_ELMAN) ? 16 : fused_epl(local, ncw, cell, ks, mtw) <= 2 ? 8 : 4;
}

__host__ __device__ constexpr int fused_hpad(bool f32) { return f32 ? 4 : 8; }
// gated tiles per compute wave (NCW compute waves, K split KS ways, MTW tiles per wave)
__host__ __device__ constexpr int fused_gt(int ncw, int ks, int mtw) {
  return ks == 1 ? mtw : (mtw * (ncw / ks) + ncw - 1) / ncw;
}
__host__ __device__ constexpr int fused_threads(int ncw) { return (ncw + 1) * 64; }

struct FusedLds {
  int h, part, wx, out, dma, r, total;
};

// A whole bf16 Elman head per workgroup streams Wx straight into LDS (global_load_lds): a ring of
// FUSED_DMA_STAGES steps, each slot FUSED_DMA_NE x 64 dwords in load order (dword i of load e at
// slot + 4 (64 e + i): row b, units 2j, 2j+1 at dword b * D/2 + j). Nothing is held in registers
// across steps, so no wait of the I/O wave covers more than the one step it needs.
constexpr int FUSED_DMA_STAGES = 16;
constexpr int FUSED_DMA_NE = 4;  // loads per step (a row is D/2 dwords; BR * D <= 512 here)
__host__ __device__ constexpr bool fused_dma(bool local, bool f32, int cell) { return local && !f32 && cell == CELL_ELMAN; }

// s_sleep units (64 clocks) before a step's first poll round. Polls compete with the stores
// they wait for; holding back the first, certainly useless, round measured best at 4-6 units
// (D=768 B=16: 1.35 -> 1.29 us per step), while pauses between later rounds only added latency.
#ifndef FRNN_POLL_SLEEP0
#define FRNN_POLL_SLEEP0 5
#endif


// Batch rows per group of the die-local design (bounds the polling registers).
constexpr int FUSED_DIE_MAX_BR = 4;

// K-split partial sums are exchanged packed: only the first BR of the 16 MFMA batch columns are
// real, so a wave moves the real columns of its MTW tiles next to each other in every 16-lane row
// (tile j, column c at position j*BRP + c) before writing them to LDS. BRP is the column stride
// of the packing, and bounds the batch rows per group of the design.
__host__ __device__ constexpr int fused_brp(int ks, int mtw) {
  return (ks * 4 <= 16 && mtw * 4 <= 16) ? 4 : (ks * 2 <= 16 && mtw * 2 <= 16) ? 2 : 1;
}
// f32x4 entries per wave's row of packed partials: 64 and BRP of padding. The gather that follows
// the barrier reads, for 16-lane row c = k2 * BRP + cc, entry k2 * row + cc: with a row of 64 + BRP
// entries that is 64 k2 + c, so consecutive lanes read consecutive 16-byte entries modulo the 256
// words of a full row set and no two lanes of a read share a bank (with 65 entries lanes
// (k2, cc + 1) and (k2 + 1, cc) met on one bank when BRP = 2).
__host__ __device__ constexpr int fused_part_row(int ks, int mtw) { return 64 + fused_brp(ks, mtw); }
// Most batch rows per group a die-local design takes.
__host__ __device__ constexpr int fused_max_br(int ks, int mtw) {
  return ks > 1 ? (fused_brp(ks, mtw) < FUSED_DIE_MAX_BR ? fused_brp(ks, mtw) : FUSED_DIE_MAX_BR) : FUSED_DIE_MAX_BR;
}

// Words (units) one lane polls per load: 16 bytes where that takes fewer loads per lane than 8
// bytes (measured: D=768 B=16, 1.32 -> 1.21 us per step), else 8 (wider loads on fewer lanes
// measured 1-3 % slower where the count of loads is the same).
__host__ __device__ constexpr int fused_poll_words(int ks, int mtw, int ktw) {
  return (fused_max_br(ks, mtw) * ktw * 16 + 63) / 64 > (fused_max_br(ks, mtw) * ktw * 8 + 63) / 64 ? 4 : 2;
}

// Byte offsets of the LDS regions (identical on host and device).
// Words (32-bit, two bf16 units each) per row of a compute wave's poll stage, padded by 16 bytes.
__host__ __device__ constexpr int fused_stage_row(int ktw) { return ktw * 16 + 4; }

// ktl: k-tiles per compute wave whose R^T fragments live in LDS instead of VGPRs (a head too wide
// for the die's registers), 1 KB per (wave, tile, k-tile) after the other regions.
__host__ __device__ inline FusedLds fused_lds(bool local, bool f32, int ncw, int ks, int mtw, int D, int cell,
                                              int ktl = 0) {
  FusedLds L;
  const int gt = fused_gt(ncw, ks, mtw);
  const int mt_wg = mtw * (ncw / ks);
  const int ktw = D / (f32 ? 4 : 32) / ks;
  L.h = 0;
  // LOCAL: the h buffer; die-local: each compute wave's poll stage, 16 rows
  const int hbytes = local ? 2 * 16 * (D + fused_hpad(f32)) * (f32 ? 4 : 2) : ncw * 16 * fused_stage_row(ktw) * 4;
  L.part = (hbytes + 15) & ~15;
  const int pbytes = (!local && ks > 1) ? 2 * ncw * fused_part_row(ks, mtw) * 16 : 0;
  L.wx = L.part + pbytes;
  L.out = L.wx + 2 * ncw * gt * 1024;
  L.dma = L.out + 2 * ncw * gt * 1024;
  L.r = L.dma + (fused_dma(local, f32, cell) ? FUSED_DMA_STAGES * FUSED_DMA_NE * 256 : 0);
  L.total = L.r + ncw * mtw * ktl * 1024;
  return L;
}

__device__ __forceinline__ void block_barrier() { __syncthreads(); }

// DPP lane moves within 16-lane rows. row_shr:n makes lane l read lane l-n of its row, row_shl:n
// lane l+n; a lane outside the bank mask, or whose source falls outside the row, keeps `old`
// (or reads 0 with bound_ctrl).
// Place columns 0..BRP-1 of tiles J..MTW-1 of acc at row positions j*BRP + c of P, in increasing
// j: positions below j*BRP keep what earlier tiles put there (their source lane is outside the
// row), positions above are overwritten by later tiles or unused.
template <int BRP, int J, int MTW>
__device__ __forceinline__ void pack_tiles(f32x4_t& P, const f32x4_t (&acc)[MTW]) {
  if constexpr (J < MTW) {
    constexpr int sh = J * BRP;
    constexpr int b0 = sh / 4, b1 = (sh + BRP - 1) / 4;
    constexpr int bank = ((1 << (b1 + 1)) - 1) & ~((1 << b0) - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      P[i] = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(P[i]), __float_as_int(acc[J][i]),
                                                        0x110 + sh, 0xF, bank, false));
    pack_tiles<BRP, J + 1, MTW>(P, acc);
  }
}

// x[p] += x[p + d] for d = D, 2D, ... < LIM within each row (positions past the row read 0):
// position c ends up with the sum over positions c + m*D.
template <int D, int LIM>
__device__ __forceinline__ void row_reduce(f32x4_t& x) {
  if constexpr (D < LIM) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[i] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[i]), 0x100 + D, 0xF, 0xF, true));
    row_reduce<2 * D, LIM>(x);
  }
}

// A flag every lane reads the same, as a wave-uniform value: branches on it stay scalar, so loops
// that leave on it keep a plain structure (and the compiler's count of loads in flight exact).
__device__ __forceinline__ bool uniform_flag(int v) { return __builtin_amdgcn_readfirstlane(v) != 0; }


// Poll the exchange words of one compute wave's K range (KTW k-tiles of 32 words from word k0 of
// each row, rows row_words apart) for rows 0 .. nvalid-1, with all 64 lanes and PW words per lane
// and load (PW = fused_poll_words), until every word carries `tag`; then unpack the values (the
// words' high halves) into the wave's LDS stage, row r at r * fused_stage_row(KTW) words, two
// bf16 per word, from which the MFMA B fragments are read. The loads bypass the CU cache (cache
// policy sc1, the coherence of an agent-scope atomic load). Each 32-bit word carries its own tag,
// so a load that sees some words of this step and some of the last is simply polled again. A
// lane without a load of its own re-reads the first one and checks nothing, so that no load sits
// under a lane mask and neither the check nor the unpacking needs a branch. Every wait is bounded: past timeout_ticks of
// the wall clock, or once another workgroup has raised an error, the wave records a timeout and
// sets *abort_flag (every wave then leaves after the next barrier).
template <int KS, int MTW, int KTW>
__device__ __forceinline__ void poll_stage(const uint32_t* xbase, int xbytes, int soff, int row_words, int k0,
                                           int nvalid, uint32_t tag, bool first_step, uint32_t* stage, int lane,
                                           long long timeout_ticks, int* err, int* abort_flag) {
  constexpr int PW = fused_poll_words(KS, MTW, KTW);
  constexpr int WPR = KTW * 32 / PW;                            // loads per row
  constexpr int NP = (fused_max_br(KS, MTW) * WPR + 63) / 64;  // loads per lane (bound)
  constexpr int SROW = fused_stage_row(KTW);
  typedef uint32_t pw_t __attribute__((ext_vector_type(PW)));
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(xbase), (short)0, xbytes, 0x00020000);
  const int nw = nvalid * WPR;
  int voff[NP], sidx[NP];
  uint32_t tmask[NP];
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    const int wi = lane + 64 * e, r = wi / WPR, wr = wi - r * WPR;
    const bool ok = wi < nw;
    voff[e] = ((ok ? r * row_words + wr * PW : 0) + k0) * 4;
    tmask[e] = ok ? 0xFFFFu : 0u;
    // a lane without a load writes its (unused) values into the padding words at the end of a
    // stage row, which no fragment read touches, so that the writes need no branch (measured
    // 1.213 -> 1.202 us per step at LSTM B=16 D=768)
    sidx[e] = ok ? r * SROW + wr * (PW / 2) : (lane & 15) * SROW + KTW * 16;
  }
  pw_t v[NP];
  long long t_first = 0;
  int spins = 0;
  // nothing can have arrived yet (a store takes a few hundred ns to show on another CU)
  if (!first_step) __builtin_amdgcn_s_sleep(FRNN_POLL_SLEEP0);
  while (true) {
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      if constexpr (PW == 4) v[e] = __builtin_amdgcn_raw_buffer_load_b128(xr, voff[e], soff, 16);
      else v[e] = __builtin_amdgcn_raw_buffer_load_b64(xr, voff[e], soff, 16);
    }
    uint32_t bad = 0;
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      uint32_t x = 0;
#pragma unroll
      for (int i = 0; i < PW; ++i) x |= v[e][i] ^ tag;
      bad |= x & tmask[e];
    }
    if (__all(bad == 0)) {
#pragma unroll
      for (int e = 0; e < NP; ++e) {
        if constexpr (PW == 4)
          *reinterpret_cast<uint2*>(stage + sidx[e]) = make_uint2(pack_hi(v[e][0], v[e][1]), pack_hi(v[e][2], v[e][3]));
        else
          stage[sidx[e]] = pack_hi(v[e][0], v[e][1]);
      }
      return;
    }
    if ((++spins & 63) == 0) {
      const long long now = (long long)wall_clock64();
      if (t_first == 0) t_first = now;
      if (now - t_first > timeout_ticks ||
          uniform_flag(__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
        if (lane == 0) atomicOr(err, DEVERR_TIMEOUT);
        *abort_flag = 1;
        return;
      }
    }
  }
}

// ---------------------------------------------------------------------------- I/O wave
// Everything the I/O wave needs, as plain values (no reference to the kernel argument).
struct IoCtx {
  const char* wxb;
  int wx_f32;
  long long wx_sb, wx_st;
  float* out_h;
  float* out_c;
  long long out_sb, out_st;
  int b0, nvalid, n, N, D, T, U_wg, u_base, lane;
};

// Float index, in slot 0 of an LDS ring, of hidden unit u (local to the workgroup) of batch column
// b and gate g: the compute lane, wave and gated-tile slot that own it, and the component of the
// lane's f32x4.
template <int CELL, int NCW, int KS, int MTW, int GT>
__device__ __forceinline__ int io_ring_float(int b, int g, int u) {
  int tq, ln, comp;
  if (cell_slots(CELL) == 4) { tq = u >> 2; ln = b + 16 * (u & 3); comp = g; }
  else { tq = u >> 4; ln = b + 16 * ((u & 15) >> 2); comp = u & 3; }
  const int wv = (KS == 1) ? tq / MTW : (tq % NCW);
  const int q = (KS == 1) ? tq % MTW : (tq / NCW);
  return ((wv * GT + q) * 64 + ln) * 4 + comp;
}

// Per-lane descriptors of the I/O wave, computed once. The Wx of one step for the workgroup is
// nvalid x G x U_wg elements (u fastest), read as 64-bit words (4 bf16 or 2 fp32 each, so that
// consecutive lanes read consecutive addresses); the outputs of one step are nvalid x U_wg
// (h and, for the LSTM, c), written as pairs of floats.
template <int CELL, int NCW, int KS, int MTW, int EPL>
struct IoDesc {
  static constexpr int G = cell_gates(CELL);
  static constexpr int GT = fused_gt(NCW, KS, MTW);
  static constexpr int E = EPL;
  // consecutive units of one word land 16 lanes apart (LSTM, GRU) or in consecutive components
  // (Elman)
  static constexpr int USTEP = (cell_slots(CELL) == 4) ? 64 : 1;
  long long wofs[E];  // byte offset of the word for step 0
  int wlds[E];        // float index of its first element in slot 0 of the Wx ring (-1: none)
  long long oofs[E];  // element offset of the output pair for step 0
  int olds[E];        // float index of its first element in slot 0 of the output ring (-1: none)
  int epw;            // elements per 64-bit word

  __device__ __forceinline__ void init(const IoCtx& c) {
    epw = c.wx_f32 ? 2 : 4;
    const int esz = c.wx_f32 ? 4 : 2;
    const int wpr = c.U_wg / epw;  // words per (b, g) row of Wx
    const int ppr = c.U_wg / 2;    // output pairs per row b
    const int nw = c.nvalid * G * wpr;
    const int no = c.nvalid * ppr;
    // word index lane + 64 e, walked incrementally (one division per lane, not per element)
    int row = c.lane / wpr, uw = c.lane - row * wpr;
    int orow = c.lane / ppr, ou = c.lane - orow * ppr;
    // a lane without a word of its own reloads the workgroup's first word, so that every load is
    // unconditional (a load under a lane mask makes the compiler wait for it on the spot)
    const long long w0 = ((long long)c.b0 * c.wx_sb + (long long)c.n * c.D + c.u_base) * esz;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int wi = c.lane + 64 * e;
      wlds[e] = -1;
      wofs[e] = w0;
      if (wi < nw) {
        const int g = row % G, b = row / G;
        const int u = uw * epw;
        wofs[e] = ((long long)(c.b0 + b) * c.wx_sb + (long long)(g * c.N + c.n) * c.D + c.u_base + u) * esz;
        wlds[e] = io_ring_float<CELL, NCW, KS, MTW, GT>(b, g, u);
      }
      olds[e] = -1;
      oofs[e] = 0;
      if (wi < no) {
        const int u = ou * 2;
        oofs[e] = (long long)(c.b0 + orow) * c.out_sb + (long long)c.n * c.D + c.u_base + u;
        olds[e] = io_ring_float<CELL, NCW, KS, MTW, GT>(orow, 0, u);
      }
      uw += 64;
      while (uw >= wpr) { uw -= wpr; ++row; }
      ou += 64;
      while (ou >= ppr) { ou -= ppr; ++orow; }
    }
  }
};

typedef uint32_t io_word_t __attribute__((ext_vector_type(2)));

template <int CELL, int NCW, int KS, int MTW, int EPL>
__device__ __forceinline__ void io_issue(const IoCtx& c, const IoDesc<CELL, NCW, KS, MTW, EPL>& d, int s,
                                         io_word_t (&r)[EPL]) {
  const long long step = (long long)s * c.wx_st * (c.wx_f32 ? 4 : 2);
#pragma unroll
  for (int e = 0; e < EPL; ++e) r[e] = *reinterpret_cast<const io_word_t*>(c.wxb + d.wofs[e] + step);
}

template <int CELL, int NCW, int KS, int MTW, int EPL>
__device__ __forceinline__ void io_put(const IoCtx& c, const IoDesc<CELL, NCW, KS, MTW, EPL>& d, int s,
                                       const io_word_t (&r)[EPL], f32x4_t* wxs) {
  typedef IoDesc<CELL, NCW, KS, MTW, EPL> Dd;
  float* wf = reinterpret_cast<float*>(wxs) + (s & 1) * (NCW * Dd::GT * 64 * 4);
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int i = d.wlds[e];
    if (i >= 0) {
      if (c.wx_f32) {
        wf[i] = __uint_as_float(r[e][0]);
        wf[i + Dd::USTEP] = __uint_as_float(r[e][1]);
      } else {
        wf[i] = __uint_as_float(r[e][0] << 16);
        wf[i + Dd::USTEP] = __uint_as_float(r[e][0] & 0xFFFF0000u);
        wf[i + 2 * Dd::USTEP] = __uint_as_float(r[e][1] << 16);
        wf[i + 3 * Dd::USTEP] = __uint_as_float(r[e][1] & 0xFFFF0000u);
      }
    }
  }
}

template <int CELL, int NCW, int KS, int MTW, int EPL>
__device__ __forceinline__ void io_store(const IoCtx& c, const IoDesc<CELL, NCW, KS, MTW, EPL>& d, int s, const f32x4_t* outs) {
  typedef IoDesc<CELL, NCW, KS, MTW, EPL> Dd;
  const float* of = reinterpret_cast<const float*>(outs) + (s & 1) * (NCW * Dd::GT * 64 * 4);
  const long long step = (long long)s * c.out_st;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int i = d.olds[e];
    if (i >= 0) {
      const long long o = d.oofs[e] + step;
      // h is component 0 (LSTM, c is component 1) of the owning lane; Elman units are components
      if (c.out_h) {
        float2 hv;
        hv.x = of[i];
        hv.y = of[i + Dd::USTEP];
        *reinterpret_cast<float2*>(c.out_h + o) = hv;
      }
      if (CELL == CELL_LSTM && c.out_c) {
        float2 cv;
        cv.x = of[i + 1];
        cv.y = of[i + Dd::USTEP + 1];
        *reinterpret_cast<float2*>(c.out_c + o) = cv;
      }
    }
  }
}

// One ring stage: interval k writes Wx of step k+1-G0 into LDS (and refills the stage with step
// k+1-G0+L), stores the outputs of step k-1-G0, then joins the step's barrier.
template <int CELL, int NCW, int KS, int MTW, int EPL, int G0, int L, int ST>
__device__ __forceinline__ bool io_interval(const IoCtx& c, const IoDesc<CELL, NCW, KS, MTW, EPL>& d, int k,
                                            io_word_t (&raw)[L][EPL], f32x4_t* wxs,
                                            const f32x4_t* outs, const int* abort_flag) {
  const int s_wx = k + 1 - G0;
  if (s_wx >= 0 && s_wx < c.T) io_put<CELL, NCW, KS, MTW, EPL>(c, d, s_wx, raw[ST], wxs);
  // Every interval issues the same loads (outside the range the step is clamped and the reload
  // is never used), so that the compiler can count the loads in flight on every path and wait
  // for the one L intervals back only.
  io_issue<CELL, NCW, KS, MTW, EPL>(c, d, min(max(s_wx + L, 0), c.T - 1), raw[ST]);
  const int s_out = k - 1 - G0;
  // (single-workgroup designs, G0 == 0: the compute waves store the states themselves)
  if (G0 == 1 && s_out >= 0 && s_out < c.T) io_store<CELL, NCW, KS, MTW, EPL>(c, d, s_out, outs);
  block_barrier();
  return uniform_flag(*abort_flag);
}

// Intervals k + J .. k + L - 1 (TAIL: only those up to T). Interval k + j uses stage
// (j - G0) mod L, which holds the Wx step that interval writes. Returns true on abort.
template <int CELL, int NCW, int KS, int MTW, int EPL, int G0, int L, int J, bool TAIL>
__device__ __forceinline__ bool io_intervals(const IoCtx& c, const IoDesc<CELL, NCW, KS, MTW, EPL>& d, int k,
                                             io_word_t (&raw)[L][EPL], f32x4_t* wxs, const f32x4_t* outs,
                                             const int* abort_flag) {
  if constexpr (J < L) {
    constexpr int ST = ((J - G0) % L + L) % L;
    if (TAIL && k + J > c.T) return false;
    if (io_interval<CELL, NCW, KS, MTW, EPL, G0, L, ST>(c, d, k + J, raw, wxs, outs, abort_flag)) return true;
    return io_intervals<CELL, NCW, KS, MTW, EPL, G0, L, J + 1, TAIL>(c, d, k, raw, wxs, outs, abort_flag);
  }
  return false;
}

// The I/O wave: runs barriers -1 .. T in step with the compute waves (see the kernel), with L
// Wx steps in flight.
template <int CELL, int NCW, int KS, int MTW, int EPL, int G0, int L>
__device__ __forceinline__ void io_wave(const IoCtx& c, f32x4_t* wxs, const f32x4_t* outs, const int* abort_flag) {
  IoDesc<CELL, NCW, KS, MTW, EPL> d;
  d.init(c);
  io_word_t raw[L][EPL];
  if (c.T == 0) {  // intervals -1 and 0: the compute waves' two barriers, nothing to move
    block_barrier();
    block_barrier();
    return;
  }
  // k runs -1 .. T; the stage of the Wx step written in interval k is (k + 1 - G0) mod L, and
  // stage s first holds step s. The first loads go out in the stage order of intervals -1 ..
  // L - 2, as they do in the loop, so that the loop is entered with the same loads in flight.
#pragma unroll
  for (int j = 0; j < L; ++j) {
    const int st = ((j - G0) % L + L) % L;
    io_issue<CELL, NCW, KS, MTW, EPL>(c, d, min(st, c.T - 1), raw[st]);
  }
  // Whole groups of L intervals in the loop (no exit inside the body, so every path into an
  // interval has the same loads in flight), then at most L - 1 more.
  int k = -1;
  for (; k + L - 1 <= c.T; k += L)
    if (io_intervals<CELL, NCW, KS, MTW, EPL, G0, L, 0, false>(c, d, k, raw, wxs, outs, abort_flag)) return;
  if (io_intervals<CELL, NCW, KS, MTW, EPL, G0, L, 0, true>(c, d, k, raw, wxs, outs, abort_flag)) return;
  if (G0 == 1 && c.T >= 1) io_store<CELL, NCW, KS, MTW, EPL>(c, d, c.T - 1, outs);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector-memory operations remain
// (expcnt and lgkmcnt left alone).
__host__ __device__ constexpr int vmcnt_imm(int n) { return (n & 0xF) | (7 << 4) | (0xF << 8) | ((n >> 4) << 14); }

// The I/O wave of a single-workgroup bf16 Elman design (see FUSED_DMA_STAGES). It runs barriers
// -1 .. T with the compute waves. Interval k issues the loads of step k - 1 + L into the slot of
// step k - 1 (read by the compute waves during step k - 1, before barrier k - 1), then waits for
// the loads of step k + 1, issued L - 2 intervals earlier, and joins barrier k: the compute waves
// read step k + 1's slot after it. Every interval issues the same FUSED_DMA_NE loads (steps are
// clamped; lanes without a dword reload the first one into a slot position nobody reads), so a
// constant count of loads stays in flight. It touches no LDS itself and uses a plain s_barrier,
// so no wait of the compiler's joins its own. Single-workgroup designs never set the abort flag.
__device__ __forceinline__ void io_wave_dma(const char* wxb, long long wx_sb, long long wx_st, int b0, int nvalid,
                                            int n, int D, int T, int lane, char* ring) {
  constexpr int L = FUSED_DMA_STAGES, NE = FUSED_DMA_NE;
  const int dpr = D / 2;  // dwords per batch row
  long long goff[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int wi = lane + 64 * e, r = wi / dpr, j = wi - r * dpr;
    goff[e] = r < nvalid ? ((long long)(b0 + r) * wx_sb + (long long)n * D) * 2 + 4LL * j
                         : ((long long)b0 * wx_sb + (long long)n * D) * 2;
  }
  const long long step_bytes = wx_st * 2;
  auto issue = [&](int s) {
    const int sc = min(max(s, 0), T - 1);
    char* slot = ring + (s & (L - 1)) * NE * 256;
#pragma unroll
    for (int e = 0; e < NE; ++e)
      __builtin_amdgcn_global_load_lds((glb_void_t*)(wxb + goff[e] + sc * step_bytes), (lds_void_t*)(slot + 256 * e), 4, 0, 0);
  };
  if (T == 0) {
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_barrier();
    return;
  }
  for (int s = 0; s <= L - 3; ++s) issue(s);
  for (int k = -1; k <= T; ++k) {
    issue(k - 1 + L);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((L - 2) * NE));
    __builtin_amdgcn_s_barrier();
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load may land after the workgroup has ended
}

template <int CELL, bool F32, bool LOCAL, int NCW, int KS, int MTW, int KTW, int KTL = 0>
__global__ void __launch_bounds__((NCW + 1) * 64, 1) fused_fwd_kernel(FusedArgs a) {
  constexpr int NT = (NCW + 1) * 64;
  constexpr int MS = NCW / KS;
  constexpr int MT_WG = MTW * MS;
  constexpr int KW = F32 ? 4 : 32;
  constexpr int GT = fused_gt(NCW, KS, MTW);
  constexpr int G = cell_gates(CELL);    // gates stored in Wx, R, b
  constexpr int GS = cell_slots(CELL);   // rows of a unit in a tile
  constexpr bool QUAD = GS == 4;         // a lane gates one unit (LSTM, GRU) or four (Elman)
  constexpr int UPT = QUAD ? 4 : 16;     // hidden units per tile
  constexpr int G0 = LOCAL ? 0 : 1;                  // gating of step s happens in interval s + G0
  static_assert((NCW == 4 || NCW == 6 || NCW == 8) && NCW % KS == 0, "compute waves / K split");
  static_assert(!(F32 && !LOCAL), "fp32 runs only in the workgroup-local design");
  static_assert(!(LOCAL && KS != 1), "the workgroup-local design does not split K");
  // the last KTL of a wave's KTW k-tiles keep their R^T fragments in LDS (die-local bf16 only)
  static_assert(KTL == 0 || (!LOCAL && !F32 && KTL < KTW), "R^T in LDS: die-local bf16 designs");
  constexpr int KTR = KTW - KTL;  // k-tiles whose fragments stay in VGPRs
  typedef typename std::conditional<F32, float, bf16x8_t>::type frag_t;

  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int s_abort;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, quad = lane >> 4;
  const int D = a.D, N = a.N, T = a.T;
  const int TPH = (GS * D) / 16;

  int group, w;
  if (LOCAL) {
    group = blockIdx.x;
    w = 0;
  } else {
    // the group is formed from the workgroups that landed on one die (see die_position)
    const int pos = die_position(a.xcc_of, a.n_xcd, a.ctr, a.slots, a.err);
    if (pos < 0) return;
    const int die = pos % a.n_xcd, slot = pos / a.n_xcd;
    group = (slot / a.W) * a.n_xcd + die;
    w = slot % a.W;
  }
  if (group >= a.groups) return;
  if (threadIdx.x == 0) s_abort = 0;

  const int n = group % N, bblk = group / N;
  const int b0 = bblk * a.BR;
  const int nvalid = min(a.BR, a.B - b0);
  const int tile0 = w * MT_WG;
  const FusedLds lay = fused_lds(LOCAL, F32, NCW, KS, MTW, D, CELL, KTL);
  constexpr int HPAD = fused_hpad(F32);
  const int HS = D + HPAD;  // row stride of the LDS h buffer (elements)
  float* hbuf_f = reinterpret_cast<float*>(smem + lay.h);
  uint16_t* hbuf_b = reinterpret_cast<uint16_t*>(smem + lay.h);
  f32x4_t* part = reinterpret_cast<f32x4_t*>(smem + lay.part);
  f32x4_t* wxs = reinterpret_cast<f32x4_t*>(smem + lay.wx);
  f32x4_t* outs = reinterpret_cast<f32x4_t*>(smem + lay.out);

  // zero the Wx ring (lanes of padding batch columns read zeros) and, for LOCAL, write
  // h_{-1} (the initial state) into parity 1 of the LDS h buffer
  for (int i = threadIdx.x; i < 2 * NCW * GT * 64; i += NT) wxs[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (!LOCAL) {  // poll stages: rows of padding batch columns stay zero
    uint32_t* st = reinterpret_cast<uint32_t*>(smem + lay.h);
    for (int i = threadIdx.x; i < NCW * 16 * fused_stage_row(KTW); i += NT) st[i] = 0u;
  }
  if (LOCAL) {
    for (int idx = threadIdx.x; idx < 16 * D; idx += NT) {
      const int c = idx / D, k = idx - c * D;
      float v = 0.0f;
      if (a.s0_h && c < nvalid) v = ld_f(a.s0_h, (long long)(b0 + c) * a.s0_sb + (long long)n * a.s0_sn + k, a.s0_f32);
      if (F32) {
        hbuf_f[(1 * 16 + c) * HS + k] = v;
        hbuf_f[c * HS + k] = 0.0f;
      } else {
        hbuf_b[(1 * 16 + c) * HS + k] = f2bf(v);
        hbuf_b[c * HS + k] = 0;
      }
    }
  }
  // A whole Elman head with at most four batch rows: only columns 0-3 of the MFMA result are
  // real, so before the gates the four units of lane (quad, column b) move to lanes (quad,
  // 4 i + b), one unit per lane, and a quarter of the transcendentals remain on the chain
  // (Elman D=128: 0.565 -> 0.512 us per step; B=16 N=12 D=64: 0.299 -> 0.287).
  const bool narrow = (CELL == CELL_ELMAN) && LOCAL && !F32 && a.BR <= 4;

  const int u_base = tile0 * UPT;                   // first hidden unit of this workgroup
  const int U_wg = min(MT_WG * UPT, D - u_base);    // its hidden units (the last tiles may be idle)

  // Time direction of this head: a head that runs backwards reads Wx and writes its states
  // from step T-1 down, through the same strides negated.
  const bool rev = n >= a.rev_n0;
  const long long wx_st = rev ? -a.wx_st : a.wx_st, out_st = rev ? -a.out_st : a.out_st;
  const char* const wx0 = reinterpret_cast<const char*>(a.Wx) + (rev ? (long long)(T - 1) * a.wx_st * (a.wx_f32 ? 4 : 2) : 0);
  float* const out_h = a.out_h ? a.out_h + (rev ? (long long)(T - 1) * a.out_st : 0) : nullptr;
  float* const out_c = a.out_c ? a.out_c + (rev ? (long long)(T - 1) * a.out_st : 0) : nullptr;

  constexpr bool DMA = fused_dma(LOCAL, F32, CELL);
  char* const dring = smem + lay.dma;
  if constexpr (DMA) {
    if (wave == NCW) {
      io_wave_dma(wx0, a.wx_sb, wx_st, b0, nvalid, n, D, T, lane, dring);
      return;
    }
  }
  if (wave == NCW) {
    IoCtx c;
    c.wxb = wx0;
    c.wx_f32 = a.wx_f32;
    c.wx_sb = a.wx_sb;
    c.wx_st = wx_st;
    c.out_h = out_h;
    c.out_c = out_c;
    c.out_sb = a.out_sb;
    c.out_st = out_st;
    c.b0 = b0;
    c.nvalid = nvalid;
    c.n = n;
    c.N = N;
    c.D = D;
    c.T = T;
    c.U_wg = U_wg;
    c.u_base = u_base;
    c.lane = lane;
    io_wave<CELL, NCW, KS, MTW, fused_epl(LOCAL, NCW, CELL, KS, MTW), G0, fused_io_stages(LOCAL, NCW, CELL, KS, MTW)>(c, wxs, outs, &s_abort);
    return;
  }

  // ==================================================================== compute waves
  const int ks = wave % KS, ms = wave / KS;
  const bool colv = col < nvalid;
  const long long bcol = b0 + col;
  const bool r_f32 = F32;

  // ---- R^T fragments, resident for the whole sequence. bf16: 16 contiguous bytes per lane from
  // the packed copy, all loads in flight at once (tiles past the head read its last tile and are
  // zeroed).
  frag_t Ra[MTW][KTR];
  // the LDS-resident fragments of this wave: [tile j][k-tile kk - KTR][64 lanes], 16 bytes a lane
  u32x4_t* const rl = reinterpret_cast<u32x4_t*>(smem + lay.r) + (long long)wave * MTW * (KTL > 0 ? KTL : 1) * 64;
  if constexpr (F32) {
#pragma unroll
    for (int j = 0; j < MTW; ++j) {
      const int tt = tile0 + ms * MTW + j;
      const bool tv = tt < TPH;
      int u, g;
      if (QUAD) { u = 4 * tt + (col >> 2); g = col & 3; }
      else { u = 16 * tt + col; g = 0; }
      const bool rv = tv && g < G;  // rows of gates the cell does not have are zero
      const long long rbase = (long long)(g < G ? g : 0) * a.r_sg + (long long)n * a.r_sn + u;
#pragma unroll
      for (int kk = 0; kk < KTW; ++kk) {
        const int k = (ks * KTW + kk) * KW + quad;
        Ra[j][kk] = rv ? reinterpret_cast<const float*>(a.R)[rbase + (long long)k * a.r_sd] : 0.0f;
      }
    }
  } else {
    const int KT = D / 32;
    const u32x4_t* rp = reinterpret_cast<const u32x4_t*>(a.rpack) + (long long)n * TPH * KT * 64 + lane;
    u32x4_t raw[MTW][KTR];
#pragma unroll
    for (int j = 0; j < MTW; ++j) {
      const int tt = min(tile0 + ms * MTW + j, TPH - 1);
#pragma unroll
      for (int kk = 0; kk < KTR; ++kk) raw[j][kk] = rp[((long long)tt * KT + ks * KTW + kk) * 64];
    }
#pragma unroll
    for (int j = 0; j < MTW; ++j) {
      const bool tv = tile0 + ms * MTW + j < TPH;
#pragma unroll
      for (int kk = 0; kk < KTR; ++kk) {
        u32x4_t v = raw[j][kk];
        if (!tv) v = u32x4_t{0u, 0u, 0u, 0u};
        Ra[j][kk] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
    if constexpr (KTL > 0) {  // the rest go to LDS, read back every step (the first barrier orders them)
#pragma unroll
      for (int j = 0; j < MTW; ++j) {
        const int tr = tile0 + ms * MTW + j;
        const int tt = min(tr, TPH - 1);
#pragma unroll
        for (int kk = KTR; kk < KTW; ++kk) {
          u32x4_t v = rp[((long long)tt * KT + ks * KTW + kk) * 64];
          if (tr >= TPH) v = u32x4_t{0u, 0u, 0u, 0u};
          rl[(j * KTL + (kk - KTR)) * 64 + lane] = v;
        }
      }
    }
  }

  // ---- tiles this wave applies the gates to, their bias and initial state (LSTM c; GRU h,
  // kept in fp32 for the update while the MFMA operand is its bf16 copy).
  int gu[GT];  // LSTM, GRU: the lane's unit; Elman: first of the lane's four units
  bool gval[GT];
  float bia[GT][4], creg[GT];
#pragma unroll
  for (int q = 0; q < GT; ++q) {
    const int tq = (KS == 1) ? ms * MTW + q : wave + NCW * q;
    const int tt = tile0 + tq;
    gval[q] = (tq < MT_WG) && (tt < TPH);
    gu[q] = QUAD ? 4 * tt + quad : 16 * tt + 4 * quad;
    creg[q] = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) bia[q][i] = 0.0f;
    if (gval[q]) {
      if (a.bias) {
#pragma unroll
        for (int i = 0; i < (QUAD ? G : 4); ++i) {
          const long long off = QUAD ? (long long)(i * N + n) * D + gu[q] : (long long)n * D + gu[q] + i;
          bia[q][i] = ld_f(a.bias, off, r_f32);
        }
      }
      if (CELL == CELL_LSTM && a.s0_c && colv)
        creg[q] = ld_f(a.s0_c, bcol * a.s0_sb + (long long)n * a.s0_sn + gu[q], a.s0_f32);
      if (CELL == CELL_GRU && a.s0_h && colv)
        creg[q] = ld_f(a.s0_h, bcol * a.s0_sb + (long long)n * a.s0_sn + gu[q], a.s0_f32);
    }
  }
  block_barrier();  // barrier -1

  // exchange words of this group: uniform base (scalar registers) plus 32-bit lane offsets
  uint32_t* const xb = a.xbuf + (long long)group * 2 * a.BR * D;
  const int xpar = a.BR * D;  // words per parity
  // The initial h of this workgroup's units goes out like any later step's h: parity 1, tag 0 (the
  // buffer starts filled with tag 0xFFFF), so step 0 polls it like every other step.
  if (!LOCAL && !F32 && colv) {
#pragma unroll
    for (int q = 0; q < GT; ++q) {
      if (!gval[q]) continue;
#pragma unroll
      for (int i = 0; i < (QUAD ? 1 : 4); ++i) {
        const int u = gu[q] + i;
        const float h0 = a.s0_h ? ld_f(a.s0_h, bcol * a.s0_sb + (long long)n * a.s0_sn + u, a.s0_f32) : 0.0f;
        xb[xpar + col * D + u] = (uint32_t)f2bf(h0) << 16;
      }
    }
  }
  float hlast[GT][4];         // h of the last step, written out after the loop

  for (int t = 0; t < T; ++t) {
    // Wx of this step (the ring slot t & 1, written by the I/O wave before the barrier that
    // precedes the gating): read as early as that barrier allows
    f32x4_t wxq[GT];
    if constexpr (DMA) {
      // four units of row col from the DMA ring: two dwords (rows past nvalid read the last row)
      const uint32_t* slot = reinterpret_cast<const uint32_t*>(dring + (t & (FUSED_DMA_STAGES - 1)) * FUSED_DMA_NE * 256);
      const int rb = min(col, nvalid - 1);
#pragma unroll
      for (int q = 0; q < GT; ++q) {
        const uint2 w = *reinterpret_cast<const uint2*>(slot + rb * (D / 2) + (gval[q] ? gu[q] / 2 : 0));
        wxq[q] = f32x4_t{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                         __uint_as_float(w.y & 0xFFFF0000u)};
      }
    } else if (LOCAL) {
#pragma unroll
      for (int q = 0; q < GT; ++q) wxq[q] = wxs[(((t & 1) * NCW + wave) * GT + q) * 64 + lane];
    }
    // Keep those reads here, ahead of the MFMAs: the compiler would otherwise sink them into the
    // gating branch that uses them, after the MFMAs, and put their LDS latency on the step's chain.
    if (LOCAL) asm volatile("" ::: "memory");
    // ---- 1+2. h_{t-1} as the B operand, multiplied on MFMA as each k-tile becomes available.
    f32x4_t acc[MTW];
#pragma unroll
    for (int j = 0; j < MTW; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (LOCAL) {
      const int p = (t + 1) & 1;
#pragma unroll
      for (int kk = 0; kk < KTW; ++kk) {
        frag_t bk;
        if constexpr (F32) bk = hbuf_f[(p * 16 + col) * HS + kk * KW + quad];
        else bk = *reinterpret_cast<const bf16x8_t*>(&hbuf_b[(p * 16 + col) * HS + kk * KW + 8 * quad]);
#pragma unroll
        for (int j = 0; j < MTW; ++j) {
          if constexpr (F32) acc[j] = mfma_f32(Ra[j][kk], bk, acc[j]);
          else acc[j] = mfma_bf16(Ra[j][kk], bk, acc[j]);
        }
      }
    } else if constexpr (!F32) {
      // this wave's K range of h_{t-1}, polled into the wave's LDS stage
      uint32_t* stage = reinterpret_cast<uint32_t*>(smem + lay.h) + wave * 16 * fused_stage_row(KTW);
      poll_stage<KS, MTW, KTW>(xb, 2 * xpar * 4, ((t - 1) & 1) * xpar * 4, D, ks * KTW * 32, nvalid,
                               (uint32_t)t & 0xFFFFu, t == 0, stage, lane, a.timeout_ticks, a.err, &s_abort);
#pragma unroll
      for (int kk = 0; kk < KTW; ++kk) {
        const bf16x8_t bk = *reinterpret_cast<const bf16x8_t*>(stage + col * fused_stage_row(KTW) + kk * 16 + 4 * quad);
#pragma unroll
        for (int j = 0; j < MTW; ++j) {
          if constexpr (KTL > 0) {
            if (kk >= KTR) {
              const bf16x8_t ak = __builtin_bit_cast(bf16x8_t, rl[(j * KTL + (kk - KTR)) * 64 + lane]);
              acc[j] = mfma_bf16(ak, bk, acc[j]);
              continue;
            }
          }
          acc[j] = mfma_bf16(Ra[j][kk < KTR ? kk : 0], bk, acc[j]);
        }
      }
    }

    // ---- 3. (die-local design) the step's barrier; K-split partial sums through LDS.
    f32x4_t pre[GT];
    if constexpr (KS == 1) {
#pragma unroll
      for (int q = 0; q < GT; ++q) pre[q] = acc[q];
      if (!LOCAL) {
        block_barrier();
#pragma unroll
        for (int q = 0; q < GT; ++q) wxq[q] = wxs[(((t & 1) * NCW + wave) * GT + q) * 64 + lane];
        if (uniform_flag(s_abort)) return;
      }
    } else {
      // pack the real batch columns of this wave's MTW tiles into one f32x4 per lane and write it;
      // after the barrier one read gathers, for each tile this wave gates, the KS partials of
      // its columns (source k2, column c at row position k2*BRP + c), and row_reduce adds them
      constexpr int BRP = fused_brp(KS, MTW);
      constexpr int PROW = fused_part_row(KS, MTW);
      const int pp = t & 1;
      f32x4_t P = acc[0];
      pack_tiles<BRP, 1, MTW>(P, acc);
      part[(pp * NCW + wave) * PROW + lane] = P;
      block_barrier();
      // the reads go out before the abort flag is looked at (they are harmless if it is set)
#pragma unroll
      for (int q = 0; q < GT; ++q) wxq[q] = wxs[(((t & 1) * NCW + wave) * GT + q) * 64 + lane];
      const int k2 = col / BRP, cc = col - k2 * BRP;
#pragma unroll
      for (int q = 0; q < GT; ++q) {
        pre[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int tq = wave + NCW * q;
        const int msq = tq / MTW, jq = tq - msq * MTW;
        if (gval[q] && k2 < KS)
          pre[q] = part[(pp * NCW + msq * KS + k2) * PROW + quad * 16 + jq * BRP + cc];
      }
      if (uniform_flag(s_abort)) return;
#pragma unroll
      for (int q = 0; q < GT; ++q) row_reduce<BRP, KS * BRP>(pre[q]);
    }

    // ---- 4. gates, state update, exchange; outputs go to the LDS ring for the I/O wave.
    // The step the host names in stall_step (a failure-handling test; -1 in every normal call)
    // publishes the tag of step t - 1, which no consumer polls for, so that their bounded waits
    // run out and every workgroup leaves through the abort path.
    const uint32_t wtag = (uint32_t)(t + 1 - (t == a.stall_step ? 2 : 0)) & 0xFFFFu;
#pragma unroll
    for (int q = 0; q < GT; ++q) {
      if (!gval[q]) continue;
      const int ri = (((t & 1) * NCW + wave) * GT + q) * 64 + lane;
      const f32x4_t wx4 = wxq[q];
      if constexpr (QUAD) {
        float h, c = 0.0f;
        if constexpr (CELL == CELL_LSTM) {
          const float ig = sigmoid_f(pre[q][0] + wx4[0] + bia[q][0]);
          const float fg = sigmoid_f(pre[q][1] + wx4[1] + bia[q][1]);
          const float zg = tanh_f(pre[q][2] + wx4[2] + bia[q][2]);
          const float og = sigmoid_f(pre[q][3] + wx4[3] + bia[q][3]);
          c = fg * creg[q] + ig * zg;
          creg[q] = c;
          h = og * tanh_f(c);
        } else {  // GRU: the reset gate scales the candidate's recurrent part only
          const float rg = sigmoid_f(pre[q][0] + wx4[0] + bia[q][0]);
          const float zg = sigmoid_f(pre[q][1] + wx4[1] + bia[q][1]);
          const float ng = tanh_f(wx4[2] + rg * (pre[q][2] + bia[q][2]));
          h = ng + zg * (creg[q] - ng);  // (1 - z) n + z h
          creg[q] = h;
        }
        const int u = gu[q];
        if (LOCAL) {
          if constexpr (F32) hbuf_f[((t & 1) * 16 + col) * HS + u] = h;
          else hbuf_b[((t & 1) * 16 + col) * HS + u] = f2bf(h);
          // no global load is ever waited for in these waves, so the state stores cost no wait
          if (colv) {
            const long long o = bcol * a.out_sb + (long long)t * out_st + (long long)n * D + u;
            if (out_h) out_h[o] = h;
            if (CELL == CELL_LSTM && out_c) out_c[o] = c;
          }
        } else {
          if (colv) xb[(t & 1) * xpar + col * D + u] = ((uint32_t)f2bf(h) << 16) | wtag;
          outs[ri] = f32x4_t{h, c, 0.f, 0.f};
        }
        hlast[q][0] = h;
      } else if (CELL == CELL_ELMAN && LOCAL && !F32 && narrow) {
        f32x4_t y;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = pre[q][i] + wx4[i] + bia[q][i];
        // lane 16 quad + 4 i + b takes component i of lane 16 quad + b (row shifts by 4 i, written
        // only into bank i of each 16-lane row)
        float x = y[0];
        x = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(y[1]), 0x114, 0xF, 0x2, false));
        x = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(y[2]), 0x118, 0xF, 0x4, false));
        x = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(y[3]), 0x11C, 0xF, 0x8, false));
        const float hv = tanh_f(x);
        const int bb = col & 3, u1 = gu[q] + (col >> 2);
        hbuf_b[((t & 1) * 16 + bb) * HS + u1] = f2bf(hv);
        if (bb < nvalid && out_h) out_h[(long long)(b0 + bb) * a.out_sb + (long long)t * out_st + (long long)n * D + u1] = hv;
        hlast[q][0] = hv;
      } else {
        float h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = tanh_f(pre[q][i] + wx4[i] + bia[q][i]);
        const int u = gu[q];
        if (LOCAL) {
          if constexpr (F32) {
            *reinterpret_cast<f32x4_t*>(&hbuf_f[((t & 1) * 16 + col) * HS + u]) = f32x4_t{h[0], h[1], h[2], h[3]};
          } else {
            u16x4_t hv = {f2bf(h[0]), f2bf(h[1]), f2bf(h[2]), f2bf(h[3])};
            *reinterpret_cast<u16x4_t*>(&hbuf_b[((t & 1) * 16 + col) * HS + u]) = hv;
          }
          if (colv && out_h)
            *reinterpret_cast<f32x4_t*>(out_h + bcol * a.out_sb + (long long)t * out_st + (long long)n * D + u) =
                f32x4_t{h[0], h[1], h[2], h[3]};
        } else {
          if (colv) {
            u32x4_t wv;
#pragma unroll
            for (int i = 0; i < 4; ++i) wv[i] = ((uint32_t)f2bf(h[i]) << 16) | wtag;
            *reinterpret_cast<u32x4_t*>(xb + ((t & 1) * xpar + col * D + u)) = wv;
          }
          outs[ri] = f32x4_t{h[0], h[1], h[2], h[3]};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) hlast[q][i] = h[i];
      }
    }
    // Keep the exchange stores ahead of the next step's polling in program order.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (LOCAL) block_barrier();
  }
  block_barrier();  // barrier T: the last step's outputs are in LDS for the I/O wave
  // last_states: the state after the last step, straight from registers
  if (T > 0 && narrow) {
    const int bb = col & 3;
#pragma unroll
    for (int q = 0; q < GT; ++q)
      if (gval[q] && bb < nvalid && a.last_h)
        a.last_h[(long long)(b0 + bb) * a.last_sb + (long long)n * a.last_sn + gu[q] + (col >> 2)] = hlast[q][0];
  } else if (T > 0 && colv) {
#pragma unroll
    for (int q = 0; q < GT; ++q) {
      if (!gval[q]) continue;
      const long long lo = bcol * a.last_sb + (long long)n * a.last_sn + gu[q];
      if constexpr (QUAD) {
        if (a.last_h) a.last_h[lo] = hlast[q][0];
        if (CELL == CELL_LSTM && a.last_c) a.last_c[lo] = creg[q];
      } else if (a.last_h) {
        *reinterpret_cast<f32x4_t*>(a.last_h + lo) = f32x4_t{hlast[q][0], hlast[q][1], hlast[q][2], hlast[q][3]};
      }
    }
  }
}

}  // namespace frnn
