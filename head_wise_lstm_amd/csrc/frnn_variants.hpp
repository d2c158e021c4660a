// The fused kernel's instantiated designs. Each cell's instantiations live in a translation unit
// of their own (frnn_fused_<cell>.hip), so that the three compile in parallel; the host planner
// looks designs up in the tables those units export.
#pragma once

#include "frnn_fused.hpp"
#include "frnn_fused_bwd.hpp"

namespace frnn {

typedef void (*fused_fn)(FusedArgs);

struct FusedVariant {
  int cell, f32, local, ncw, ks, mtw, ktw;
  int ktl;  // k-tiles per compute wave whose R^T fragments live in LDS (0: all in VGPRs)
  fused_fn fn;
};

struct FusedTable {
  const FusedVariant* v;
  int n;
};

// X(F32, LOCAL, NCW, KS, MTW, KTW): (compute waves, K split, tiles per wave, k-tiles per wave).
// Each fits the register file without spilling at its wave count (checked with
// -Rpass-analysis=kernel-resource-usage).
#define FRNN_FUSED_DESIGNS(X)                                                                      \
  /* die-local multi-workgroup design (bf16) */                                                    \
  X(false, false, 4, 4, 1, 1) X(false, false, 4, 4, 2, 1) X(false, false, 4, 4, 1, 2)              \
  X(false, false, 4, 4, 2, 2) X(false, false, 4, 4, 3, 3) X(false, false, 4, 4, 4, 4)              \
  X(false, false, 4, 4, 2, 4) X(false, false, 4, 4, 4, 2) X(false, false, 4, 4, 4, 1)              \
  X(false, false, 4, 2, 1, 1) X(false, false, 4, 2, 2, 1) X(false, false, 4, 2, 1, 2)              \
  X(false, false, 4, 2, 2, 2) X(false, false, 4, 1, 1, 1) X(false, false, 4, 1, 1, 2)              \
  X(false, false, 8, 8, 6, 3) X(false, false, 8, 8, 4, 2) X(false, false, 8, 8, 2, 1)              \
  X(false, false, 6, 6, 6, 4) X(false, false, 4, 4, 6, 6) X(false, false, 8, 8, 8, 2)              \
  X(false, false, 4, 4, 8, 4) X(false, false, 8, 8, 4, 1) X(false, false, 8, 4, 4, 4)              \
  X(false, false, 8, 8, 2, 4)                                                                      \
  /* single-workgroup design (bf16) */                                                             \
  X(false, true, 4, 1, 1, 1) X(false, true, 4, 1, 2, 1) X(false, true, 4, 1, 1, 2)                 \
  X(false, true, 4, 1, 4, 2) X(false, true, 4, 1, 6, 3) X(false, true, 4, 1, 2, 4)                 \
  X(false, true, 4, 1, 1, 4)                                                                       \
  /* single-workgroup design (fp32) */                                                             \
  X(true, true, 4, 1, 2, 8) X(true, true, 4, 1, 1, 8) X(true, true, 4, 1, 4, 16)                   \
  X(true, true, 4, 1, 1, 16)

// Die-local bf16 designs that keep part of R^T in LDS: X(NCW, KS, MTW, KTW, KTL), the last KTL of a
// wave's KTW k-tiles in LDS. A head of 1024 units with four gate rows (8 MB of bf16 R^T over the 32
// workgroups of a die, 256 KB each) fits the registers of no design here: eight compute waves x
// eight tiles x three k-tiles in VGPRs (96 registers a lane), the fourth k-tile in LDS (64 KB).
#define FRNN_FUSED_RLDS_DESIGNS(X) X(8, 8, 8, 4, 1)

FusedTable fused_table_lstm();
FusedTable fused_table_elman();
FusedTable fused_table_gru();

// The fused backward's designs, per cell: X(NCW, KS, MTW, KTW) with K = G*D split KS ways.
typedef void (*fused_bwd_fn)(FusedBwdArgs);

struct FusedBwdVariant {
  int cell, ncw, ks, mtw, ktw;
  fused_bwd_fn fn;
};

struct FusedBwdTable {
  const FusedBwdVariant* v;
  int n;
};

// D = 768 (head split 24 ways), 512, 256, 128, 96 and 64
#define FRNN_FUSED_BWD_LSTM(X)                                                          \
  X(8, 8, 2, 12) X(6, 6, 2, 16) X(8, 8, 2, 8) X(8, 8, 1, 8) X(8, 8, 2, 4) X(4, 4, 2, 8) \
  X(8, 8, 1, 4) X(4, 4, 1, 8) X(8, 8, 1, 2) X(4, 4, 1, 4) X(8, 8, 2, 2) X(4, 4, 2, 4)   \
  X(4, 4, 1, 2) X(4, 4, 2, 2) X(4, 2, 1, 4) X(4, 4, 1, 3)
#define FRNN_FUSED_BWD_GRU(X)                                                           \
  X(8, 8, 2, 9) X(6, 6, 2, 12) X(8, 8, 2, 6) X(8, 8, 1, 6) X(8, 8, 2, 3) X(6, 6, 2, 4)  \
  X(8, 8, 1, 3) X(6, 6, 1, 4) X(6, 6, 1, 2) X(6, 6, 2, 2) X(4, 4, 2, 3) X(6, 6, 1, 1)   \
  X(6, 6, 2, 1) X(4, 2, 1, 3)
#define FRNN_FUSED_BWD_ELMAN(X)                                                         \
  X(8, 8, 1, 2) X(8, 8, 2, 2) X(8, 8, 1, 1) X(8, 8, 2, 1) X(4, 4, 1, 2) X(4, 4, 2, 2)   \
  X(4, 4, 1, 1) X(4, 4, 2, 1) X(4, 2, 1, 2) X(4, 2, 1, 1)

FusedBwdTable fused_bwd_table_lstm();
FusedBwdTable fused_bwd_table_elman();
FusedBwdTable fused_bwd_table_gru();

// The partial-sum backward design, per cell: X(NCW, MTW, KTW) with NCW * MTW = D / 16 row tiles
// and KTW * 32 = G * D / W (the workgroup's unit slice with all its gates).
#define FRNN_FUSED_BWDX_LSTM(X)                                                                       \
  X(8, 6, 3) X(6, 8, 3) X(8, 4, 2) X(8, 4, 4) X(4, 8, 2) X(8, 2, 1) X(8, 2, 2) X(8, 2, 4) \
  X(4, 4, 2) X(4, 4, 4) X(8, 1, 1) X(8, 1, 2) X(8, 1, 4) X(4, 2, 1) X(4, 2, 2) X(4, 2, 4) X(4, 1, 1) \
  X(4, 1, 2) X(4, 1, 4) X(6, 1, 2) X(6, 1, 4)
#define FRNN_FUSED_BWDX_GRU(X) \
  X(8, 6, 3) X(8, 4, 3) X(8, 2, 3) X(4, 4, 3) X(8, 1, 3) X(4, 2, 3) X(4, 1, 3) X(6, 1, 3)
#define FRNN_FUSED_BWDX_ELMAN(X)                                                                      \
  X(8, 6, 1) X(8, 4, 1) X(8, 2, 1) X(4, 4, 1) X(8, 1, 1) X(4, 2, 1) X(8, 1, 2) X(4, 2, 2) X(4, 1, 1)
// Partial-sum designs X(NCW, MTW, KTW, KTL) that keep the last KTL of a wave's k-tiles of R in LDS:
// heads of 1024 units, whose slice of R (32 units with all their gates, all 1024 rows) fits the
// VGPRs of no design without spilling (nine waves leave 168 VGPRs a lane). LSTM: two of four
// k-tiles in LDS (with one, the step's MFMA phase spills); GRU: one of three.
#define FRNN_FUSED_BWDX_RLDS_LSTM(X) X(8, 8, 4, 2)
#define FRNN_FUSED_BWDX_RLDS_GRU(X) X(8, 8, 3, 1)

struct FusedBwdxVariant {
  int cell, ncw, mtw, ktw, ktl;
  fused_bwd_fn fn;
};

struct FusedBwdxTable {
  const FusedBwdxVariant* v;
  int n;
};

FusedBwdxTable fused_bwdx_table_lstm();
FusedBwdxTable fused_bwdx_table_elman();
FusedBwdxTable fused_bwdx_table_gru();

// The single-workgroup backward (fused_bwd_local_kernel) of a cell for heads of D units, D = 32 or
// 64 (its k-tiles, G*D/4 on the fp32 MFMA or G*D/32 on the bf16 one where bf, are a template
// parameter), or null for any other D.
fused_bwd_fn fused_bwd_local_lstm(int D, bool bf);
fused_bwd_fn fused_bwd_local_elman(int D, bool bf);
fused_bwd_fn fused_bwd_local_gru(int D, bool bf);

}  // namespace frnn
