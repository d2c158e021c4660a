// Persistent fused backward recurrence (the serial part of back-propagation through time) for
// gfx950.
//
// Once the forward's states are known, every step's gates are known, and the backward of a step
// is linear in the two gradients it carries (dh, and the LSTM's dc) with per-element coefficients
// that depend only on the step. Those coefficients are computed for all steps at once beforehand
// (bwd_record_kernel), so the serial part is a linear recurrence:
//   LSTM:  dh = dh_R + ds_h;  dc = dc' + ds_c + dh*A1;  da = (dc*A2, dc*A3, dc*A4, dh*A5);  dc' <- dc*A6
//   GRU:   dh = dh_R + ds_h + dh';  da = (dh*C1, dh*C2, dh*C4);  dh' <- dh*C5
//   Elman: dh = dh_R + ds_h;  da = dh*E1
//   dh_R of the step before = sum_g da_g . R_g^T
// (ds_h, ds_c: the gradients of the step's outputs). Steps run in reverse: step s of the kernel is
// timestep t = T-1-s.
//
// The kernel is the forward's die-local design with the roles of h and R^T exchanged: the W
// workgroups of a group (one head, BR batch rows, one die) each own 16-unit tiles of R's rows d,
// resident in VGPRs for all steps, with k = (g, e) over G*D. Lane l of an MFMA result holds
// dh_R of units 4*(l/16)..+3 of its tile for batch column l%16, applies the step to them, and
// publishes their da (G words per unit, bf16 << 16 | step tag) through the die's L2; every
// workgroup polls the da of the whole group (its K range per wave) as the next step's B operand.
// A fifth kind of wave, the I/O wave, streams the step records into an LDS ring ahead of the
// steps (this design: four steps ahead through registers, and it writes each step's (dh, dc) out
// of another ring; the partial-sum and single-workgroup designs below: LDS-direct loads, with
// (dh, dc) stored by the lanes that compute them). dWx and the dR operand are formed from (dh,
// dc) afterwards, for all steps at once (bwd_post_kernel).
#pragma once

#include "frnn_fused.hpp"

namespace frnn {

// floats per (step, batch row, head, unit) record:
//   LSTM  [A1 A2 A3 A4 | A5 A6 ds_h ds_c]
//   GRU   [C1 C2 C4 C5 | ds_h C3 0 0]
//   Elman [E1 ds_h 0 0 | 0 0 0 0]
constexpr int BWD_REC = 8;
constexpr int BWD_EPL_IN = 8;   // 64-bit record words one I/O lane moves per step (at most)
constexpr int BWD_EPL_OUT = 2;  // 64-bit (dh, dc) words one I/O lane moves per step (at most)

struct FusedBwdArgs {
  int B, T, N, D;    // B: the rows of this launch (a chunk of the batch)
  int Bs;            // rows of the record and output arrays (their step stride)
  int BR, groups, W, n_xcd, slots;  // slots: workgroups on each of the n_xcd dies
  uint32_t xcc_of;   // hardware XCC id of die d in bits [4d, 4d+4)
  uint32_t* ctr;     // per-die workgroup counters (filled with 0xFFFF before the launch)
  const void* rpk;   // R as A fragments: [N][D/16][G*D/32][64] x 8 bf16 (bwd_rpack_kernel)
  const float* rec;  // [T][B][N][D][BWD_REC], indexed by the kernel step s
  float* dstate;     // [T][B][N][D][2]: (dh, dc) of kernel step s (the da design's output)
  uint32_t* xbuf;    // [groups][2][BR][G*D] exchange words
  int* err;
  long long timeout_ticks;
  int stall_step;    // a failure-handling test's hook: this step publishes a stale tag (-1: none)
  // The partial-sum and single-workgroup designs store dWx, the dR operand da (as bwd_apply lays
  // them out) and the carries of time step 0 themselves, instead of the state gradients: row b of
  // this launch is batch row bbase + b.
  int bbase;
  float* dWx;        // [B,T,G,N,D] slices (or null)
  long long wx_sb, wx_st;
  void* da;          // [N][Kp][G*D] dR operand (fp32 where f32op, else bf16)
  int Kp, f32op;
  float* carry;      // [B][N][D]
  // raw = 1: no records at all; the I/O wave loads each step's h and its state gradient ds_h
  // straight from the forward's states and the caller's gradient (or the zero page), in rows of
  // [h: D floats][ds_h: D floats], and the step's coefficients 1 - h^2 and ds_h (+ dl_h at the
  // last time step) come from them (16-byte aligned rows and strides)
  int raw;
  const float* st_h;
  const float* ds_h;  // (or null)
  const float* dl_h;  // (or null)
  const float* zeros; // 256 zero bytes
  long long st_sb, st_st, last_sb;
};

struct FusedBwdLds {
  int stage, part, rin, rout, total;
};

__host__ __device__ inline FusedBwdLds fused_bwd_lds(int ncw, int ks, int mtw, int ktw, int BR, int U) {
  FusedBwdLds L;
  L.stage = 0;
  const int sbytes = ncw * 16 * fused_stage_row(ktw) * 4;
  L.part = (sbytes + 15) & ~15;
  const int pbytes = ks > 1 ? 2 * ncw * fused_part_row(ks, mtw) * 16 : 0;
  L.rin = L.part + pbytes;
  L.rout = L.rin + 2 * BR * U * BWD_REC * 4;
  L.total = L.rout + 2 * BR * U * 2 * 4;
  return L;
}

// ---------------------------------------------------------------------------- I/O wave
// The workgroup's slice of a step's records is nvalid rows of U*BWD_REC contiguous floats, and
// its (dh, dc) output nvalid rows of U*2 floats; both rings hold them densely, [row][...].
struct BwdIo {
  const char* rec;      // bytes
  float* dst;
  long long in_base, in_row, in_step;     // floats
  long long out_base, out_row, out_step;  // floats
  int nvalid, U, T, BR, lane;
  long long iofs[BWD_EPL_IN];  // float offset of the lane's record word for step 0
  int ilds[BWD_EPL_IN];        // float index in slot 0 of the input ring (-1: none)
  long long oofs[BWD_EPL_OUT];
  int olds[BWD_EPL_OUT];

  __device__ __forceinline__ void init() {
    const int wpr = U * BWD_REC / 2, opr = U;  // 64-bit words per row
#pragma unroll
    for (int e = 0; e < BWD_EPL_IN; ++e) {
      const int wi = lane + 64 * e;
      const int r = wi / wpr, w = wi - r * wpr;
      const bool ok = r < nvalid;
      iofs[e] = ok ? in_base + r * in_row + 2 * w : in_base;  // no word: reload the first one
      ilds[e] = ok ? r * U * BWD_REC + 2 * w : -1;
    }
#pragma unroll
    for (int e = 0; e < BWD_EPL_OUT; ++e) {
      const int wi = lane + 64 * e;
      const int r = wi / opr, w = wi - r * opr;
      const bool ok = r < nvalid;
      oofs[e] = ok ? out_base + r * out_row + 2 * w : 0;
      olds[e] = ok ? r * U * 2 + 2 * w : -1;
    }
  }
};

__device__ __forceinline__ void bio_issue(const BwdIo& c, int s, io_word_t (&r)[BWD_EPL_IN]) {
  const long long step = (long long)s * c.in_step * 4;
#pragma unroll
  for (int e = 0; e < BWD_EPL_IN; ++e) r[e] = *reinterpret_cast<const io_word_t*>(c.rec + c.iofs[e] * 4 + step);
}

__device__ __forceinline__ void bio_put(const BwdIo& c, int s, const io_word_t (&r)[BWD_EPL_IN], float* rin) {
  float* slot = rin + (s & 1) * (c.BR * c.U * BWD_REC);
#pragma unroll
  for (int e = 0; e < BWD_EPL_IN; ++e) {
    const int i = c.ilds[e];
    if (i >= 0) *reinterpret_cast<io_word_t*>(slot + i) = r[e];
  }
}

__device__ __forceinline__ void bio_store(const BwdIo& c, int s, const float* rout) {
  const float* slot = rout + (s & 1) * (c.BR * c.U * 2);
  const long long step = (long long)s * c.out_step;
#pragma unroll
  for (int e = 0; e < BWD_EPL_OUT; ++e) {
    const int i = c.olds[e];
    if (i >= 0) *reinterpret_cast<float2*>(c.dst + c.oofs[e] + step) = *reinterpret_cast<const float2*>(slot + i);
  }
}

// Interval k: put the records of step k into the ring, refill the stage with step k + 4, store
// the outputs of step k - 2, then join barrier k (the compute waves' step barrier).
template <int ST>
__device__ __forceinline__ bool bio_interval(const BwdIo& c, int k, io_word_t (&raw)[FUSED_IO_STAGES][BWD_EPL_IN],
                                             float* rin, const float* rout, const int* abort_flag) {
  constexpr int L = FUSED_IO_STAGES;
  if (k >= 0 && k < c.T) bio_put(c, k, raw[ST], rin);
  bio_issue(c, min(max(k + L, 0), c.T - 1), raw[ST]);  // unconditional (clamped) so every path has the same loads in flight
  if (k - 2 >= 0 && k - 2 < c.T) bio_store(c, k - 2, rout);
  block_barrier();
  return uniform_flag(*abort_flag);
}

__device__ __forceinline__ void bio_wave(BwdIo& c, float* rin, const float* rout, const int* abort_flag) {
  constexpr int L = FUSED_IO_STAGES;
  static_assert(L == 4, "the interval loop below is unrolled for four stages");
  c.init();
  io_word_t raw[L][BWD_EPL_IN];
  // stage (k mod 4) holds step k; interval -1 uses stage 3
  if (c.T == 0) {
    block_barrier();
    block_barrier();
    return;
  }
  bio_issue(c, min(3, c.T - 1), raw[3]);
  bio_issue(c, 0, raw[0]);
  bio_issue(c, min(1, c.T - 1), raw[1]);
  bio_issue(c, min(2, c.T - 1), raw[2]);
  int k = -1;
  for (; k + 3 <= c.T; k += L) {
    if (bio_interval<3>(c, k, raw, rin, rout, abort_flag)) return;
    if (bio_interval<0>(c, k + 1, raw, rin, rout, abort_flag)) return;
    if (bio_interval<1>(c, k + 2, raw, rin, rout, abort_flag)) return;
    if (bio_interval<2>(c, k + 3, raw, rin, rout, abort_flag)) return;
  }
  if (k <= c.T && bio_interval<3>(c, k, raw, rin, rout, abort_flag)) return;
  if (k + 1 <= c.T && bio_interval<0>(c, k + 1, raw, rin, rout, abort_flag)) return;
  if (k + 2 <= c.T && bio_interval<1>(c, k + 2, raw, rin, rout, abort_flag)) return;
  if (c.T >= 1) bio_store(c, c.T - 1, rout);
}

// ---------------------------------------------------------------------------- kernel
template <int CELL, int NCW, int KS, int MTW, int KTW>
__global__ void __launch_bounds__((NCW + 1) * 64, 1) fused_bwd_kernel(FusedBwdArgs a) {
  constexpr int G = cell_gates(CELL);
  constexpr int MS = NCW / KS;
  constexpr int MT_WG = MTW * MS;
  constexpr int GT = fused_gt(NCW, KS, MTW);
  static_assert((NCW == 4 || NCW == 6 || NCW == 8) && NCW % KS == 0, "compute waves / K split");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int s_abort;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, quad = lane >> 4;
  const int D = a.D, N = a.N, T = a.T;
  const int GD = G * D;
  const int TPH = D / 16;     // row tiles of a head
  const int KT = GD / 32;     // k-tiles of a head

  // the group is formed from the workgroups that landed on one die (see die_position)
  const int pos = die_position(a.xcc_of, a.n_xcd, a.ctr, a.slots, a.err);
  if (pos < 0) return;
  const int die = pos % a.n_xcd, slot = pos / a.n_xcd;
  const int group = (slot / a.W) * a.n_xcd + die;
  const int w = slot % a.W;
  if (group >= a.groups) return;
  if (threadIdx.x == 0) s_abort = 0;

  const int n = group % N, bblk = group / N;
  const int b0 = bblk * a.BR;
  const int nvalid = min(a.BR, a.B - b0);
  const int tile0 = w * MT_WG;
  const int u_base = tile0 * 16;
  const int U = MT_WG * 16;  // units of this workgroup (the planner divides the head evenly)
  const FusedBwdLds lay = fused_bwd_lds(NCW, KS, MTW, KTW, a.BR, U);
  constexpr int SROW = fused_stage_row(KTW);
  f32x4_t* part = reinterpret_cast<f32x4_t*>(smem + lay.part);
  float* rin = reinterpret_cast<float*>(smem + lay.rin);
  float* rout = reinterpret_cast<float*>(smem + lay.rout);
  {  // poll stages: rows of padding batch columns stay zero
    uint32_t* st = reinterpret_cast<uint32_t*>(smem + lay.stage);
    for (int i = threadIdx.x; i < NCW * 16 * SROW; i += (NCW + 1) * 64) st[i] = 0u;
  }

  if (wave == NCW) {
    BwdIo c;
    c.rec = reinterpret_cast<const char*>(a.rec);
    c.dst = a.dstate;
    c.in_row = (long long)N * D * BWD_REC;
    c.in_step = (long long)a.Bs * N * D * BWD_REC;
    c.in_base = ((long long)b0 * N + n) * D * BWD_REC + (long long)u_base * BWD_REC;
    c.out_row = (long long)N * D * 2;
    c.out_step = (long long)a.Bs * N * D * 2;
    c.out_base = ((long long)b0 * N + n) * D * 2 + (long long)u_base * 2;
    c.nvalid = nvalid;
    c.U = U;
    c.T = T;
    c.BR = a.BR;
    c.lane = lane;
    bio_wave(c, rin, rout, &s_abort);
    return;
  }

  // ==================================================================== compute waves
  const int ks = wave % KS, ms = wave / KS;
  const bool colv = col < nvalid;

  // ---- R fragments (rows d of this workgroup's tiles, k = (g, e) of this wave's K range)
  bf16x8_t Ra[MTW][KTW];
  {
    const u32x4_t* rp = reinterpret_cast<const u32x4_t*>(a.rpk) + (long long)n * TPH * KT * 64 + lane;
    u32x4_t raw[MTW][KTW];
#pragma unroll
    for (int j = 0; j < MTW; ++j) {
      const int tt = min(tile0 + ms * MTW + j, TPH - 1);
#pragma unroll
      for (int kk = 0; kk < KTW; ++kk) raw[j][kk] = rp[((long long)tt * KT + ks * KTW + kk) * 64];
    }
#pragma unroll
    for (int j = 0; j < MTW; ++j) {
      const bool tv = tile0 + ms * MTW + j < TPH;
#pragma unroll
      for (int kk = 0; kk < KTW; ++kk) {
        u32x4_t v = raw[j][kk];
        if (!tv) v = u32x4_t{0u, 0u, 0u, 0u};
        Ra[j][kk] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
  }

  // ---- tiles this wave applies the step to: lane (col, quad) owns units gu .. gu+3
  int gu[GT];
  bool gval[GT];
  float cr[GT][4];  // LSTM dc, GRU dh carried to the next kernel step
#pragma unroll
  for (int q = 0; q < GT; ++q) {
    const int tq = (KS == 1) ? ms * MTW + q : wave + NCW * q;
    const int tt = tile0 + tq;
    gval[q] = (tq < MT_WG) && (tt < TPH);
    gu[q] = 16 * tt + 4 * quad;
#pragma unroll
    for (int i = 0; i < 4; ++i) cr[q][i] = 0.0f;
  }
  block_barrier();  // barrier -1

  uint32_t* const xb = a.xbuf + (long long)group * 2 * a.BR * GD;
  const int xpar = a.BR * GD;  // words per parity
  // Step 0 has no dh_R: publish zero da with tag 0 (parity 1), which step 0 polls like any other.
  if (colv) {
#pragma unroll
    for (int q = 0; q < GT; ++q) {
      if (!gval[q]) continue;
#pragma unroll
      for (int g = 0; g < G; ++g)
        *reinterpret_cast<u32x4_t*>(xb + xpar + col * GD + g * D + gu[q]) = u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  for (int s = 0; s < T; ++s) {
    // ---- 1+2. da of the step before as the B operand (this wave's K range), on MFMA
    f32x4_t acc[MTW];
#pragma unroll
    for (int j = 0; j < MTW; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    {
      // this wave's K range of the step before's da, polled into the wave's LDS stage
      uint32_t* stage = reinterpret_cast<uint32_t*>(smem + lay.stage) + wave * 16 * SROW;
      poll_stage<KS, MTW, KTW>(xb, 2 * xpar * 4, ((s - 1) & 1) * xpar * 4, GD, ks * KTW * 32, nvalid,
                               (uint32_t)s & 0xFFFFu, s == 0, stage, lane, a.timeout_ticks, a.err, &s_abort);
#pragma unroll
      for (int kk = 0; kk < KTW; ++kk) {
        const bf16x8_t bk = *reinterpret_cast<const bf16x8_t*>(stage + col * SROW + kk * 16 + 4 * quad);
#pragma unroll
        for (int j = 0; j < MTW; ++j) acc[j] = mfma_bf16(Ra[j][kk], bk, acc[j]);
      }
    }

    // ---- 3. the step's barrier; K-split partial sums through LDS
    f32x4_t pre[GT];
    if constexpr (KS == 1) {
#pragma unroll
      for (int q = 0; q < GT; ++q) pre[q] = acc[q];
      block_barrier();
      if (uniform_flag(s_abort)) return;
    } else {
      constexpr int BRP = fused_brp(KS, MTW);
      const int pp = s & 1;
      f32x4_t P = acc[0];
      pack_tiles<BRP, 1, MTW>(P, acc);
      part[(pp * NCW + wave) * fused_part_row(KS, MTW) + lane] = P;
      block_barrier();
      const int k2 = col / BRP, cc = col - k2 * BRP;
#pragma unroll
      for (int q = 0; q < GT; ++q) {
        pre[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int tq = wave + NCW * q;
        const int msq = tq / MTW, jq = tq - msq * MTW;
        if (gval[q] && k2 < KS)
          pre[q] = part[(pp * NCW + msq * KS + k2) * fused_part_row(KS, MTW) + quad * 16 + jq * BRP + cc];
      }
      if (uniform_flag(s_abort)) return;
#pragma unroll
      for (int q = 0; q < GT; ++q) row_reduce<BRP, KS * BRP>(pre[q]);
    }

    // ---- 4. the linear step for the lane's four units; da out through the exchange, (dh, dc)
    // to the output ring
    // (the step the host names in stall_step publishes the tag of step s - 1, which no one polls
    // for: its consumers' bounded waits run out; -1 in every normal call)
    const uint32_t wtag = (uint32_t)(s + 1 - (s == a.stall_step ? 2 : 0)) & 0xFFFFu;
    if (colv) {
#pragma unroll
      for (int q = 0; q < GT; ++q) {
        if (!gval[q]) continue;
        const int ul = gu[q] - u_base;
        const float* rr = rin + ((s & 1) * a.BR + col) * U * BWD_REC + ul * BWD_REC;
        float* ro = rout + ((s & 1) * a.BR + col) * U * 2 + ul * 2;
        float da[G][4], dh[4], dc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4_t r0 = *reinterpret_cast<const f32x4_t*>(rr + i * BWD_REC);
          const f32x4_t r1 = *reinterpret_cast<const f32x4_t*>(rr + i * BWD_REC + 4);
          if constexpr (CELL == CELL_LSTM) {
            dh[i] = pre[q][i] + r1[2];
            dc[i] = cr[q][i] + r1[3] + dh[i] * r0[0];
            da[0][i] = dc[i] * r0[1];
            da[1][i] = dc[i] * r0[2];
            da[2 % G][i] = dc[i] * r0[3];
            da[3 % G][i] = dh[i] * r1[0];
            cr[q][i] = dc[i] * r1[1];
          } else if constexpr (CELL == CELL_GRU) {
            dh[i] = pre[q][i] + r1[0] + cr[q][i];
            dc[i] = 0.0f;
            da[0][i] = dh[i] * r0[0];
            da[1 % G][i] = dh[i] * r0[1];
            da[2 % G][i] = dh[i] * r0[2];
            cr[q][i] = dh[i] * r0[3];
          } else {
            dh[i] = pre[q][i] + r0[1];
            dc[i] = 0.0f;
            da[0][i] = dh[i] * r0[0];
          }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          u32x4_t wv;
#pragma unroll
          for (int i = 0; i < 4; ++i) wv[i] = ((uint32_t)f2bf(da[g][i]) << 16) | wtag;
          *reinterpret_cast<u32x4_t*>(xb + ((s & 1) * xpar + col * GD + g * D + gu[q])) = wv;
        }
        *reinterpret_cast<f32x4_t*>(ro) = f32x4_t{dh[0], dc[0], dh[1], dc[1]};
        *reinterpret_cast<f32x4_t*>(ro + 4) = f32x4_t{dh[2], dc[2], dh[3], dc[3]};
      }
    }
    // Keep the exchange stores ahead of the next step's polling in program order.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
  block_barrier();  // barrier T: the last step's outputs are in LDS for the I/O wave
}

}  // namespace frnn

namespace frnn {

// ============================================================================ partial-sum design
// The same linear recurrence with the work cut the other way. Workgroup w of a group owns the
// unit slice [w*UW, (w+1)*UW) (UW = D / W) with all its gates, so the step (and da) of its units
// needs nothing from other workgroups but dh_R of those units. Its compute waves multiply the
// slice's da (K = G*UW, from LDS) by the R columns of the slice for every row d of the head
// (all D/16 tiles, MTW per wave), and publish the result as a partial sum of dh_R: D words a row
// (bf16 << 16 | step tag) in the workgroup's own slot of the exchange. The next step's pollers
// read their units' words from all W slots (D words a row per workgroup, a quarter of the da
// exchange of the LSTM design above for G = 4) and add them in fp32.
//
// Per step s: poll waves (the first PW compute waves, four (row, unit quad) combinations each,
// sixteen slot chunks per combination in one 16-lane row, two 16-byte loads per lane, summed by
// four DPP row shifts) poll,
// apply the step (its records read from LDS, before the poll where the registers allow) and write
// da into the stage of parity s (bf16 B fragments [batch row][k], k = g*UW + unit) and (dh, dc) to
// memory; the step's barrier; every compute wave multiplies the stage by its R fragments and
// publishes. The stage has two parities: a workgroup's pollers wait only for the waves that own
// their units, so another wave may still read the stage of step s while step s+1 is written.
// The I/O wave loads the records of step k+1 into the LDS ring with LDS-direct loads, landed by
// barrier k (the step is applied before the barrier); the lanes that apply the step store its
// (dh, dc) themselves.

constexpr int BWDX_CPW = 4;  // (row, unit quad) combinations per poll wave
constexpr int BWDX_J = 16;   // slot chunks per combination (lanes = CPW * J = 64)
constexpr int BWDX_NP = 2;   // 16-byte loads per lane and round: W <= BWDX_J * BWDX_NP
constexpr int BWDX_MAX_W = BWDX_J * BWDX_NP;
// s_sleep units (64 clocks) before a step's first poll round (see FRNN_POLL_SLEEP0)
#ifndef FRNN_BWDX_SLEEP0
#define FRNN_BWDX_SLEEP0 FRNN_POLL_SLEEP0
#endif

// The record ring: BWDX_RING slots of BWDX_SLOT bytes, each filled by BWDX_NE 16-byte LDS-direct
// loads per I/O lane and step; a group's records of one step (BR * U * BWD_REC floats) fit a slot.
constexpr int BWDX_RING = 4;
constexpr int BWDX_NE = 4;
constexpr int BWDX_SLOT = 64 * 16 * BWDX_NE;

struct FusedBwdxLds {
  int stage, rin, r, total;
};

// ktl: k-tiles of R per compute wave kept in LDS (ncw waves of mtw row tiles, 1 KB per tile and
// k-tile) rather than in VGPRs.
__host__ __device__ inline FusedBwdxLds fused_bwdx_lds(int ktw, int BR, int U, int ncw = 0, int mtw = 0, int ktl = 0) {
  FusedBwdxLds L;
  L.stage = 0;
  L.rin = 2 * 16 * fused_stage_row(ktw) * 4;  // a multiple of 16 bytes, as the ring's loads need
  L.r = L.rin + BWDX_RING * BWDX_SLOT;
  L.total = L.r + ncw * mtw * ktl * 1024;
  (void)BR;
  (void)U;
  return L;
}

// The partial-sum design's I/O wave: it only loads. A step's records come straight into a slot of
// the LDS ring with 16-byte LDS-direct loads: lane l of load e writes slot bytes 1024 e + 16 l, so
// chunk i = 64 e + l of the group's dense [row][U * BWD_REC] records lands where the compute waves
// read it; a lane past the valid rows loads the first chunk again into a slot position no one
// reads. Interval k (k = -1 .. T-1) issues the loads of step k + BWDX_RING - 1 (clamped to T - 1)
// into its slot, whose last reader, step k - 1, finished before barrier k - 1; waits until the
// loads of step k + 1, issued two intervals earlier, have landed; and joins barrier k, after which
// the compute waves read step k + 1. Every interval issues the same four loads, so a constant
// count of them stays in flight; the wave touches no LDS itself and no load result passes through
// a register, so no wait of the compiler's joins in. Every exit waits for all loads, so that none
// lands after the workgroup has ended.
// A word of LDS read from inline asm, which waits for it in the same statement: a plain read would
// make the compiler wait for every LDS-direct load in flight first (it cannot tell that they write
// elsewhere), which would drain the ring each interval.
__device__ __forceinline__ int lds_read_word(const int* p) {
  const uint32_t off = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) int*)p;
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(off) : "memory");
  return v;
}

struct BwdxDma {
  const char* rec;                          // bytes
  long long in_base, in_row, in_step;       // floats
  int nvalid, U, T, lane;
};

__device__ __forceinline__ void biox_wave(const BwdxDma& c, char* ring, const int* abort_flag) {
  constexpr int NS = BWDX_RING, NE = BWDX_NE;
  static_assert(NS == 4, "the wait below counts the loads of the two intervals after a step's");
  if (c.T == 0) {
    block_barrier();
    return;
  }
  const int cpr = c.U * BWD_REC / 4;  // 16-byte chunks per row
  long long goff[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int i = c.lane + 64 * e, r = i / cpr, w = i - r * cpr;
    goff[e] = (r < c.nvalid ? c.in_base + r * c.in_row + 4 * w : c.in_base) * 4;
  }
  const long long step_bytes = c.in_step * 4;
  auto issue = [&](int s) {
    const int sc = min(max(s, 0), c.T - 1);
    char* slot = ring + (s & (NS - 1)) * BWDX_SLOT;
#pragma unroll
    for (int e = 0; e < NE; ++e)
      __builtin_amdgcn_global_load_lds((glb_void_t*)(c.rec + goff[e] + sc * step_bytes), (lds_void_t*)(slot + 1024 * e),
                                       16, 0, 0);
  };
  issue(0);  // steps 0 and 1, as intervals -3 and -2 would issue them
  issue(1);
  for (int k = -1; k < c.T; ++k) {
    issue(k + NS - 1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * NE));
    __builtin_amdgcn_s_barrier();
    if (uniform_flag(lds_read_word(abort_flag))) break;
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// The sum of x over the lane's 16-lane row, in every lane of the row: the lanes of each quad swap
// and add (quad_perm 1,0,3,2 then 2,3,0,1), then the halves of each 8-lane half-row and of the
// row (half-row and row mirrors). Every lane adds the same pairs, so all sixteen get the same bits.
__device__ __forceinline__ float row_allreduce_add(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, true));
  return x;
}

// xbuf: [groups][2][W][BR][D] words. NCW * MTW = D / 16; KTW * 32 = G * D / W; the last KTL of
// a wave's KTW k-tiles keep their R fragments in LDS.
template <int CELL, int NCW, int MTW, int KTW, int KTL = 0>
__global__ void __launch_bounds__((NCW + 1) * 64, 1) fused_bwdx_kernel(FusedBwdArgs a) {
  constexpr int G = cell_gates(CELL);
  static_assert(NCW == 4 || NCW == 6 || NCW == 8, "compute waves");
  static_assert(KTL >= 0 && KTL < KTW, "R k-tiles in LDS");
  constexpr int KTR = KTW - KTL;  // k-tiles whose fragments stay in VGPRs

  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int s_abort;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, quad = lane >> 4;
  const int D = a.D, N = a.N, T = a.T, W = a.W, BR = a.BR;
  const int GD = G * D;
  const int TPH = D / 16;
  const int KT = GD / 32;
  const int UW = D / W;

  // the group is formed from the workgroups that landed on one die (see die_position)
  const int pos = die_position(a.xcc_of, a.n_xcd, a.ctr, a.slots, a.err);
  if (pos < 0) return;
  const int die = pos % a.n_xcd, slot = pos / a.n_xcd;
  const int group = (slot / W) * a.n_xcd + die;
  const int w = slot % W;
  if (group >= a.groups) return;
  if (threadIdx.x == 0) s_abort = 0;

  const int n = group % N, bblk = group / N;
  const int b0 = bblk * BR;
  const int nvalid = min(BR, a.B - b0);
  const int u0 = w * UW;
  const FusedBwdxLds lay = fused_bwdx_lds(KTW, BR, UW, NCW, MTW, KTL);
  constexpr int SROW = fused_stage_row(KTW);
  uint32_t* stage = reinterpret_cast<uint32_t*>(smem + lay.stage);
  char* const ring = smem + lay.rin;
  // both stages: rows of padding batch columns stay zero
  for (int i = threadIdx.x; i < 2 * 16 * SROW; i += (NCW + 1) * 64) stage[i] = 0u;

  if (wave == NCW) {
    BwdxDma c;
    c.rec = reinterpret_cast<const char*>(a.rec);
    c.in_row = (long long)N * D * BWD_REC;
    c.in_step = (long long)a.Bs * N * D * BWD_REC;
    c.in_base = ((long long)b0 * N + n) * D * BWD_REC + (long long)u0 * BWD_REC;
    c.nvalid = nvalid;
    c.U = UW;
    c.T = T;
    c.lane = lane;
    biox_wave(c, ring, &s_abort);
    return;
  }

  // ==================================================================== compute waves
  // ---- R fragments: rows d of this wave's tiles, k = g*UW + e - u0 over the slice. Eight
  // consecutive k stay inside one gate (UW is a multiple of 8), so each fragment is one 16-byte
  // lane of the packed R (global k = g*D + e). The fragments of k-tiles KTR.. go to LDS, one
  // region per wave ([tile j][k-tile kk - KTR][64 lanes], 16 bytes a lane), and are read back every
  // step by the wave that wrote them.
  bf16x8_t Ra[MTW][KTR];
  u32x4_t* const rl = reinterpret_cast<u32x4_t*>(smem + lay.r) + wave * MTW * (KTL > 0 ? KTL : 1) * 64;
  {
    const u32x4_t* rp = reinterpret_cast<const u32x4_t*>(a.rpk) + (long long)n * TPH * KT * 64;
    u32x4_t raw[MTW][KTW];
#pragma unroll
    for (int kk = 0; kk < KTW; ++kk) {
      const int kl = kk * 32 + 8 * quad;
      const int g = kl / UW, kg = g * D + u0 + (kl - g * UW);
      const int ktg = kg >> 5, grp = (kg & 31) >> 3;
#pragma unroll
      for (int j = 0; j < MTW; ++j) {
        const int tt = wave * MTW + j;
        raw[j][kk] = rp[((long long)tt * KT + ktg) * 64 + grp * 16 + col];
      }
    }
#pragma unroll
    for (int j = 0; j < MTW; ++j) {
#pragma unroll
      for (int kk = 0; kk < KTR; ++kk) Ra[j][kk] = __builtin_bit_cast(bf16x8_t, raw[j][kk]);
#pragma unroll
      for (int kk = KTR; kk < KTW; ++kk) rl[(j * KTL + (kk - KTR)) * 64 + lane] = raw[j][kk];
    }
  }

  // ---- poll lanes: combination c (batch row r, unit quad q) in lanes 16c' .. 16c'+15, slot chunk
  // j = lane & 15 (slots j and j+16), one 16-byte load (the quad's four words) per slot
  static_assert(BWDX_J == 16 && BWDX_CPW * BWDX_J == 64, "poll lane layout");
  const int UQ = UW / 4;
  const int PW = (BR * UQ + BWDX_CPW - 1) / BWDX_CPW;
  const bool poller = wave < PW;
  const int cmb = wave * BWDX_CPW + (lane >> 4), chunk = lane & 15;
  const int pr = cmb / UQ, pq = cmb - pr * UQ;
  const bool cv = poller && cmb < BR * UQ && pr < nvalid;
  const int xpar = W * BR * D;  // words per parity
  uint32_t* const xb = a.xbuf + (long long)group * 2 * xpar;
  // byte offsets from the parity's base; a lane without a slot re-reads offset 0 and neither
  // checks nor adds what it reads (no load under a lane mask, no branch in the check or the sum)
  int off[BWDX_NP];
  uint32_t tmask[BWDX_NP], vmask[BWDX_NP];
#pragma unroll
  for (int e = 0; e < BWDX_NP; ++e) {
    const int ws = chunk + BWDX_J * e;
    const bool pv = cv && ws < W;
    off[e] = pv ? (ws * BR * D + pr * D + u0 + 4 * pq) * 4 : 0;
    tmask[e] = pv ? 0xFFFFu : 0u;
    vmask[e] = pv ? 0xFFFF0000u : 0u;
  }
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(xb, (short)0, 2 * xpar * 4, 0x00020000);
  const int ui = chunk & 3, gi = chunk >> 2;  // the lane's unit of the quad, and gate
  float cr = 0.0f;  // LSTM dc, GRU dh of unit ui carried to the next step

  // Step 0 has no dh_R: publish zero partials with tag 0 (parity 1), polled like any other step.
  if (col < nvalid) {
#pragma unroll
    for (int j = 0; j < MTW; ++j) {
      const int d0 = 16 * (wave * MTW + j) + 4 * quad;
      *reinterpret_cast<u32x4_t*>(xb + xpar + (w * BR + col) * D + d0) = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  block_barrier();  // barrier -1

  for (int s = 0; s < T; ++s) {
    // ---- A. poll this workgroup's units in every slot, add the partials, apply the step
    if (poller) {
      // this step's records of the lane's unit ui of the quad (in the ring since barrier s-1)
      const float* rr = reinterpret_cast<const float*>(ring + (s & (BWDX_RING - 1)) * BWDX_SLOT) +
                        (cv ? pr : 0) * UW * BWD_REC + (cv ? 4 * pq + ui : 0) * BWD_REC;
      f32x4_t rc[2];
      // The records go out before the poll (their latency hidden behind it) unless R k-tiles live
      // in LDS: those designs hold up to 96 VGPRs of R. They read the records after the poll.
      if constexpr (KTL == 0) {
        rc[0] = *reinterpret_cast<const f32x4_t*>(rr);
        rc[1] = *reinterpret_cast<const f32x4_t*>(rr + 4);
      }
      const uint32_t tag = (uint32_t)s & 0xFFFFu;
      // 16-byte loads that bypass the CU cache (cache policy sc1, the coherence of an agent-scope
      // atomic load); every 32-bit word carries its own tag, so a load that sees words of two
      // steps is simply polled again
      const int soff = ((s - 1) & 1) * xpar * 4;
      u32x4_t v[BWDX_NP];
      long long t_first = 0;
      int spins = 0;
      bool ok = false;
      if (s > 0) __builtin_amdgcn_s_sleep(FRNN_BWDX_SLEEP0);
      while (true) {
#pragma unroll
        for (int e = 0; e < BWDX_NP; ++e) v[e] = __builtin_amdgcn_raw_buffer_load_b128(xr, off[e], soff, 16);
        uint32_t bad = 0;
#pragma unroll
        for (int e = 0; e < BWDX_NP; ++e)
          bad |= ((v[e][0] ^ tag) | (v[e][1] ^ tag) | (v[e][2] ^ tag) | (v[e][3] ^ tag)) & tmask[e];
        if (__all(bad == 0)) {
          ok = true;
          break;
        }
        if ((++spins & 63) == 0) {
          const long long now = (long long)wall_clock64();
          if (t_first == 0) t_first = now;
          if (now - t_first > a.timeout_ticks ||
              uniform_flag(__hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
            if (lane == 0) atomicOr(a.err, DEVERR_TIMEOUT);
            s_abort = 1;  // every wave leaves after the next barrier
            break;
          }
        }
      }
      if (ok) {
        // every lane of the row gets the quad's four sums; lane (gi, ui) then applies the step to
        // unit ui and forms gate gi of da and dWx
        float sum[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sum[i] = 0.0f;
#pragma unroll
          for (int e = 0; e < BWDX_NP; ++e) sum[i] += __uint_as_float(v[e][i] & vmask[e]);
          sum[i] = row_allreduce_add(sum[i]);
        }
        if (cv) {
          f32x4_t r0, r1;
          if constexpr (KTL > 0) {
            r0 = *reinterpret_cast<const f32x4_t*>(rr);
            r1 = *reinterpret_cast<const f32x4_t*>(rr + 4);
          } else {
            r0 = rc[0];
            r1 = rc[1];
          }
          const float su = ui == 0 ? sum[0] : ui == 1 ? sum[1] : ui == 2 ? sum[2] : sum[3];
          float dag, dwg;  // gate gi of da and of dWx (they differ in the GRU's n gate)
          if constexpr (CELL == CELL_LSTM) {
            const float dh = su + r1[2];
            const float dc = cr + r1[3] + dh * r0[0];
            dag = gi == 0 ? dc * r0[1] : gi == 1 ? dc * r0[2] : gi == 2 ? dc * r0[3] : dh * r1[0];
            dwg = dag;
            cr = dc * r1[1];
          } else if constexpr (CELL == CELL_GRU) {
            const float dh = su + r1[0] + cr;
            dag = gi == 0 ? dh * r0[0] : gi == 1 ? dh * r0[1] : dh * r0[2];
            dwg = gi == 2 ? dh * r1[1] : dag;
            cr = dh * r0[3];
          } else {
            const float dh = su + r0[1];
            dag = dh * r0[0];
            dwg = dag;
          }
          if (gi < G) {
            const uint16_t dab = f2bf(dag);
            reinterpret_cast<uint16_t*>(stage + ((s & 1) * 16 + pr) * SROW)[gi * UW + 4 * pq + ui] = dab;
            // dWx and the dR operand straight to memory: these waves' next wait on memory is the
            // next step's poll, long after the stores have landed
            const long long bg = (long long)a.bbase + b0 + pr, t = T - 1 - s, u = u0 + 4 * pq + ui;
            if (a.dWx) a.dWx[bg * a.wx_sb + t * a.wx_st + ((long long)gi * N + n) * D + u] = dwg;
            reinterpret_cast<uint16_t*>(a.da)[((n * (long long)a.Kp + t * a.Bs + bg) * G + gi) * D + u] = dab;
            if (CELL != CELL_ELMAN && gi == 0 && s == T - 1) a.carry[(bg * N + n) * D + u] = cr;
          }
        }
      }
    }
    block_barrier();  // barrier s

    // ---- B. the slice's da times the R columns of the slice, for every row d; publish
    f32x4_t acc[MTW];
#pragma unroll
    for (int j = 0; j < MTW; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // the stage reads go out before the abort flag is looked at (they are harmless if it is set)
    const uint32_t* sg = stage + (s & 1) * 16 * SROW;
    // (designs with R k-tiles in LDS read each k-tile's operand where it is used)
    constexpr int KB = KTL > 0 ? 1 : KTW;
    bf16x8_t bks[KB];
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) bks[kk] = *reinterpret_cast<const bf16x8_t*>(sg + col * SROW + kk * 16 + 4 * quad);
    if (uniform_flag(s_abort)) return;
#pragma unroll
    for (int kk = 0; kk < KTW; ++kk) {
      const bf16x8_t bk = kk < KB ? bks[kk < KB ? kk : 0] : *reinterpret_cast<const bf16x8_t*>(sg + col * SROW + kk * 16 + 4 * quad);
#pragma unroll
      for (int j = 0; j < MTW; ++j) {
        if constexpr (KTL > 0) {
          if (kk >= KTR) {
            acc[j] = mfma_bf16(__builtin_bit_cast(bf16x8_t, rl[(j * KTL + (kk - KTR)) * 64 + lane]), bk, acc[j]);
            continue;
          }
        }
        acc[j] = mfma_bf16(Ra[j][kk < KTR ? kk : 0], bk, acc[j]);
      }
    }
    if (col < nvalid) {
      // (stall_step: a stale tag, as in the da design)
      const uint32_t wtag = (uint32_t)(s + 1 - (s == a.stall_step ? 2 : 0)) & 0xFFFFu;
      uint32_t* dst = xb + (s & 1) * xpar + (w * BR + col) * D;
#pragma unroll
      for (int j = 0; j < MTW; ++j) {
        u32x4_t wv;
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[i] = ((uint32_t)f2bf(acc[j][i]) << 16) | wtag;
        *reinterpret_cast<u32x4_t*>(dst + 16 * (wave * MTW + j) + 4 * quad) = wv;
      }
    }
    // Keep the exchange stores ahead of the next step's polling in program order.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
}

}  // namespace frnn

namespace frnn {

// ============================================================================ single-workgroup design
// Heads of at most 64 units: a whole head (and a block of BR batch rows) per workgroup, so the
// step's da stays in LDS (two parities) as the next step's B operand: no exchange, no bounded
// wait. Each compute wave owns one 16-row tile of R's rows d, resident in VGPRs, with k = (g, e)
// over G*D, A = R packed by bwd_rpack_kernel and B = da^T:
//   * fp32 inputs (BF = false): the fp32 MFMA's k-tiles of four (v_mfma_f32_16x16x4_f32), da
//     kept in fp32;
//   * bf16 inputs (BF = true): the bf16 MFMA's k-tiles of 32 (v_mfma_f32_16x16x32_bf16), da
//     rounded to bf16 as the die-local designs' operand is (an eighth of the MFMAs).
// Lane l of the result holds dh_R of units 4*(l/16)..+3 of its tile for batch column l%16, as in
// the die-local design, and applies the same linear step. The I/O wave streams the records into
// an LDS ring as the partial-sum design's does, and the lanes that apply a step store its dWx and
// da (one barrier per step).
constexpr int BWDL_NCW = 4;
// da row of the LDS stage: floats (fp32), or bf16 elements padded by 16 bytes (bf16)
__host__ __device__ constexpr int fused_bwdl_row(int G, int D, bool bf = false) { return bf ? G * D + 8 : G * D + 4; }
// The design's record ring: BWDX_RING slots of BWDL_SLOT bytes, BWDL_NE 16-byte LDS-direct loads
// per I/O lane and step; twice the partial-sum design's slot, so that a 64-unit head takes four
// batch rows a workgroup.
constexpr int BWDL_NE = 8;
constexpr int BWDL_SLOT = 64 * 16 * BWDL_NE;
// Floats a record in this design: an Elman cell's two coefficients alone (compact records:
// bwd_record_kernel with REC = 2, read where FRNN_BWD_ELMAN_RAW=0 pins them instead of the raw
// inputs), else BWD_REC.
__host__ __device__ constexpr int bwdl_rec(int cell) { return cell == CELL_ELMAN ? 2 : BWD_REC; }

struct FusedBwdlLds {
  int da, rin, total;
};

// A group's records of one step fit one slot of the record ring.
__host__ __device__ inline FusedBwdlLds fused_bwdl_lds(int G, int D, int BR, bool bf = false) {
  FusedBwdlLds L;
  L.da = 0;
  L.rin = 2 * 16 * fused_bwdl_row(G, D, bf) * (bf ? 2 : 4);  // a multiple of 16 bytes, as the ring's loads need
  L.total = L.rin + BWDX_RING * BWDL_SLOT;
  (void)BR;
  return L;
}

// The single-workgroup design's I/O wave: the partial-sum design's load-only ring (see biox_wave)
// with NE loads per lane and step of records of REC floats, on this design's schedule. The
// compute waves apply step s between barriers s and s + 1, so the
// records of step s land by barrier s, and interval k issues step k + BWDX_RING - 2, whose slot's
// last reader, step k - 2, finished at barrier k - 1. The design never aborts (it has no bounded
// wait), so the wave joins every barrier, -1 .. T.
template <int NE, int REC>
__device__ __forceinline__ void biol_wave(const BwdxDma& c, char* ring) {
  constexpr int NS = BWDX_RING;
  static_assert(NE * 64 * 16 <= BWDL_SLOT, "a step's loads fill at most one slot");
  static_assert(NS == 4, "the wait below counts the loads of the two intervals after a step's");
  static_assert((NS - 2) * NE < 64, "vmcnt counts at most 63 operations");
  if (c.T == 0) {
    block_barrier();
    block_barrier();
    return;
  }
  const int cpr = c.U * REC / 4;  // 16-byte chunks per row
  long long goff[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int i = c.lane + 64 * e, r = i / cpr, w = i - r * cpr;
    goff[e] = (r < c.nvalid ? c.in_base + r * c.in_row + 4 * w : c.in_base) * 4;
  }
  const long long step_bytes = c.in_step * 4;
  auto issue = [&](int s) {
    const int sc = min(max(s, 0), c.T - 1);
    char* slot = ring + (s & (NS - 1)) * BWDL_SLOT;
#pragma unroll
    for (int e = 0; e < NE; ++e)
      __builtin_amdgcn_global_load_lds((glb_void_t*)(c.rec + goff[e] + sc * step_bytes), (lds_void_t*)(slot + 1024 * e),
                                       16, 0, 0);
  };
  issue(0);  // step 0, as interval -2 would issue it
  for (int k = -1; k <= c.T; ++k) {
    issue(k + NS - 2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * NE));
    __builtin_amdgcn_s_barrier();
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// The raw-input form of the I/O wave above (an Elman cell's records replaced by their inputs): lane
// chunk i = 64 e + lane is 16 bytes of row r = i / (D / 2), h where its chunk w < D / 4, else ds_h;
// rows past the group's last load that row again. Step s reads time T - 1 - s.
template <int NE>
__device__ __forceinline__ void biol_raw_wave(const FusedBwdArgs& a, int n, int b0, int nvalid, int lane, char* ring) {
  constexpr int NS = BWDX_RING;
  static_assert(NE * 64 * 16 <= BWDL_SLOT, "a step's loads fill at most one slot");
  const int T = a.T, D = a.D;
  if (T == 0) {
    block_barrier();
    block_barrier();
    return;
  }
  const int cpr = D / 2, hc = D / 4;  // 16-byte chunks a row, of them h's
  const char* src[NE];
  long long step[NE];  // bytes from one kernel step's source to the next (a step back in time)
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int i = lane + 64 * e, r = min(i / cpr, nvalid - 1), w = i % cpr;
    const long long row = (long long)(a.bbase + b0 + r) * a.st_sb + (long long)(T - 1) * a.st_st + (long long)n * D;
    if (w < hc) {
      src[e] = reinterpret_cast<const char*>(a.st_h + row + 4 * w);
      step[e] = -a.st_st * 4;
    } else if (a.ds_h) {
      src[e] = reinterpret_cast<const char*>(a.ds_h + row + 4 * (w - hc));
      step[e] = -a.st_st * 4;
    } else {
      src[e] = reinterpret_cast<const char*>(a.zeros) + 16 * (w - hc);
      step[e] = 0;
    }
  }
  auto issue = [&](int s) {
    const int sc = min(max(s, 0), T - 1);
    char* slot = ring + (s & (NS - 1)) * BWDL_SLOT;
#pragma unroll
    for (int e = 0; e < NE; ++e)
      __builtin_amdgcn_global_load_lds((glb_void_t*)(src[e] + sc * step[e]), (lds_void_t*)(slot + 1024 * e), 16, 0, 0);
  };
  issue(0);  // step 0, as interval -2 would issue it
  for (int k = -1; k <= T; ++k) {
    issue(k + NS - 2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * NE));
    __builtin_amdgcn_s_barrier();
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// Largest batch rows per group: a step's records (D units a row, BWD_REC floats a unit) fill at most
// one ring slot; compact records then take a quarter of the slot's loads.
__host__ __device__ constexpr int fused_bwdl_max_br(int D) { return BWDL_SLOT / (D * BWD_REC * 4); }

template <int CELL, int KT, bool BF>
__global__ void __launch_bounds__((BWDL_NCW + 1) * 64, 1) fused_bwd_local_kernel(FusedBwdArgs a) {
  constexpr int G = cell_gates(CELL);
  constexpr int NCW = BWDL_NCW;
  constexpr int REC = bwdl_rec(CELL);  // floats a record
  constexpr bool ELM = CELL == CELL_ELMAN;  // the cell whose records may be read raw
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, quad = lane >> 4;
  const int D = a.D, N = a.N, T = a.T;
  const int TPH = D / 16;  // row tiles of a head (at most NCW)
  const int group = blockIdx.x;
  if (group >= a.groups) return;
  const int n = group % N, bblk = group / N;
  const int b0 = bblk * a.BR;
  const int nvalid = min(a.BR, a.B - b0);
  const FusedBwdlLds lay = fused_bwdl_lds(G, D, a.BR, BF);
  const int ROW = fused_bwdl_row(G, D, BF);  // elements of a da row (fp32, or bf16)
  float* dab = reinterpret_cast<float*>(smem + lay.da);
  uint16_t* dabh = reinterpret_cast<uint16_t*>(smem + lay.da);
  char* const ring = smem + lay.rin;
  // both parities of da start at zero: step 0 has no dh_R, and rows of padding batch columns
  // are never written
  for (int i = threadIdx.x; i < 2 * 16 * ROW * (BF ? 1 : 2) / 2; i += (NCW + 1) * 64) dab[i] = 0.0f;

  if (wave == NCW) {
    if (ELM && a.raw) {
      biol_raw_wave<BWDL_NE * REC / BWD_REC>(a, n, b0, nvalid, lane, ring);
      return;
    }
    BwdxDma c;
    c.rec = reinterpret_cast<const char*>(a.rec);
    c.in_row = (long long)N * D * REC;
    c.in_step = (long long)a.Bs * N * D * REC;
    c.in_base = ((long long)b0 * N + n) * D * REC;
    c.nvalid = nvalid;
    c.U = D;
    c.T = T;
    c.lane = lane;
    biol_wave<BWDL_NE * REC / BWD_REC, REC>(c, ring);
    return;
  }

  // ==================================================================== compute waves
  const bool colv = col < nvalid;
  const int tt = wave;  // the wave's tile of R's rows
  const bool tv = tt < TPH;
  // R's A fragments: KT k-tiles of 4 (fp32) or 32 (bf16) of the wave's tile
  typedef typename std::conditional<BF, bf16x8_t, float>::type afrag_t;
  afrag_t Ra[KT];
  {
    const afrag_t* rp = reinterpret_cast<const afrag_t*>(a.rpk) + ((long long)n * TPH + min(tt, TPH - 1)) * KT * 64 + lane;
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) Ra[kk] = rp[(long long)kk * 64];
  }
  const int gu = 16 * tt + 4 * quad;  // the lane's first unit
  float cr[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // LSTM dc, GRU dh carried to the next kernel step
  // raw inputs: the gradient of last_states joins ds_h at the last time step (kernel step 0)
  f32x4_t dl = {0.f, 0.f, 0.f, 0.f};
  if (ELM && a.raw && a.dl_h && colv && tv)
    dl = *reinterpret_cast<const f32x4_t*>(a.dl_h + (long long)(a.bbase + b0 + col) * a.last_sb + (long long)n * D + gu);
  block_barrier();  // barrier -1

  for (int s = 0; s < T; ++s) {
    block_barrier();  // barrier s: the step before's da and this step's records are in LDS
    if (tv) {  // (uniform in the wave; every wave reaches every barrier)
      // ---- dh_R = sum over k of R[d][k] da[k] for this wave's 16 rows d, all batch columns
      f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BF) {  // lane (col, quad): da[col][32 kk + 8 quad ..+7]
        const uint16_t* bp = dabh + ((s + 1) & 1) * 16 * ROW + col * ROW + 8 * quad;
#pragma unroll
        for (int kk = 0; kk < KT; kk += 2) {
          acc0 = mfma_bf16(Ra[kk], *reinterpret_cast<const bf16x8_t*>(bp + kk * 32), acc0);
          if (kk + 1 < KT) acc1 = mfma_bf16(Ra[kk + 1], *reinterpret_cast<const bf16x8_t*>(bp + (kk + 1) * 32), acc1);
        }
      } else {  // lane (col, quad): da[col][4 kk + quad]
        const float* bp = dab + ((s + 1) & 1) * 16 * ROW + col * ROW + quad;
#pragma unroll
        for (int kk = 0; kk < KT; kk += 2) {
          acc0 = mfma_f32(Ra[kk], bp[kk * 4], acc0);
          if (kk + 1 < KT) acc1 = mfma_f32(Ra[kk + 1], bp[(kk + 1) * 4], acc1);
        }
      }
      const f32x4_t pre = acc0 + acc1;
      if (colv) {
        // ---- the linear step for the lane's four units; da into this step's parity, (dh, dc) out
        const float* rr = reinterpret_cast<const float*>(ring + (s & (BWDX_RING - 1)) * BWDL_SLOT) + col * D * REC +
                          gu * REC;
        // dWx, da and the carries straight to memory: these waves never wait on memory
        float da[G][4], dh[4], dc[4], dwn[4];  // dwn: the GRU's n-gate dWx (its da differs)
        f32x4_t rc[2];  // compact records: the four units' (r0[0], r0[1]) pairs
        if constexpr (REC == 2) {
          if (a.raw) {  // row col of the slot: h, then ds_h, D floats each
            const float* rw = reinterpret_cast<const float*>(ring + (s & (BWDX_RING - 1)) * BWDL_SLOT) + col * 2 * D + gu;
            const f32x4_t hv = *reinterpret_cast<const f32x4_t*>(rw);
            f32x4_t dv = *reinterpret_cast<const f32x4_t*>(rw + D);
            if (s == 0) dv += dl;
            rc[0] = f32x4_t{1.0f - hv[0] * hv[0], dv[0], 1.0f - hv[1] * hv[1], dv[1]};
            rc[1] = f32x4_t{1.0f - hv[2] * hv[2], dv[2], 1.0f - hv[3] * hv[3], dv[3]};
          } else {
            rc[0] = *reinterpret_cast<const f32x4_t*>(rr);
            rc[1] = *reinterpret_cast<const f32x4_t*>(rr + 4);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4_t r0, r1;
          if constexpr (REC == 2) {
            r0 = f32x4_t{rc[i >> 1][2 * (i & 1)], rc[i >> 1][2 * (i & 1) + 1], 0.0f, 0.0f};
            r1 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
          } else {
            r0 = *reinterpret_cast<const f32x4_t*>(rr + i * REC);
            r1 = *reinterpret_cast<const f32x4_t*>(rr + i * REC + 4);
          }
          if constexpr (CELL == CELL_LSTM) {
            dh[i] = pre[i] + r1[2];
            dc[i] = cr[i] + r1[3] + dh[i] * r0[0];
            da[0][i] = dc[i] * r0[1];
            da[1][i] = dc[i] * r0[2];
            da[2 % G][i] = dc[i] * r0[3];
            da[3 % G][i] = dh[i] * r1[0];
            cr[i] = dc[i] * r1[1];
          } else if constexpr (CELL == CELL_GRU) {
            dh[i] = pre[i] + r1[0] + cr[i];
            dc[i] = 0.0f;
            da[0][i] = dh[i] * r0[0];
            da[1 % G][i] = dh[i] * r0[1];
            da[2 % G][i] = dh[i] * r0[2];
            dwn[i] = dh[i] * r1[1];
            cr[i] = dh[i] * r0[3];
          } else {
            dh[i] = pre[i] + r0[1];
            dc[i] = 0.0f;
            da[0][i] = dh[i] * r0[0];
          }
        }
        if constexpr (BF) {
          uint16_t* dw = dabh + (s & 1) * 16 * ROW + col * ROW + gu;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            uint2 v;
            v.x = (uint32_t)f2bf(da[g][0]) | ((uint32_t)f2bf(da[g][1]) << 16);
            v.y = (uint32_t)f2bf(da[g][2]) | ((uint32_t)f2bf(da[g][3]) << 16);
            *reinterpret_cast<uint2*>(dw + g * D) = v;
          }
        } else {
          float* dw = dab + (s & 1) * 16 * ROW + col * ROW + gu;
#pragma unroll
          for (int g = 0; g < G; ++g)
            *reinterpret_cast<f32x4_t*>(dw + g * D) = f32x4_t{da[g][0], da[g][1], da[g][2], da[g][3]};
        }
        const long long bg = (long long)a.bbase + b0 + col, t = T - 1 - s;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const bool nw = CELL == CELL_GRU && g == 2;
          const f32x4_t wv = nw ? f32x4_t{dwn[0], dwn[1], dwn[2], dwn[3]} : f32x4_t{da[g][0], da[g][1], da[g][2], da[g][3]};
          // (a unit quad of dWx is 16-byte aligned: the boundary takes aligned pointers and
          // strides of whole multiples of four elements)
          if (a.dWx) *reinterpret_cast<f32x4_t*>(a.dWx + bg * a.wx_sb + t * a.wx_st + ((long long)g * N + n) * D + gu) = wv;
          const long long drow = (((long long)n * a.Kp + t * a.Bs + bg) * G + g) * D + gu;
          if (a.f32op) {
            *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(a.da) + drow) = f32x4_t{da[g][0], da[g][1], da[g][2], da[g][3]};
          } else {
            uint2 w;
            w.x = (uint32_t)f2bf(da[g][0]) | ((uint32_t)f2bf(da[g][1]) << 16);
            w.y = (uint32_t)f2bf(da[g][2]) | ((uint32_t)f2bf(da[g][3]) << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.da) + drow) = w;
          }
        }
        // the carries past time step 0 (the initial state's gradient adds them)
        if (CELL != CELL_ELMAN && s == T - 1)
          *reinterpret_cast<f32x4_t*>(a.carry + (bg * N + n) * D + gu) = f32x4_t{cr[0], cr[1], cr[2], cr[3]};
      }
    }
  }
  block_barrier();  // barrier T (the I/O wave joins barriers -1 .. T)
}

}  // namespace frnn
