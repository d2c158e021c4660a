// Instantiations of the fused forward and backward kernels for the lstm cell (one translation
// unit per cell).
#include "frnn_variants.hpp"

namespace frnn {
namespace {

#define FRNN_FV(F32, LOCAL, NCW, KS, MTW, KTW) \
  {CELL_LSTM, F32, LOCAL, NCW, KS, MTW, KTW, 0, &fused_fwd_kernel<CELL_LSTM, F32, LOCAL, NCW, KS, MTW, KTW>},
#define FRNN_FVL(NCW, KS, MTW, KTW, KTL) \
  {CELL_LSTM, false, false, NCW, KS, MTW, KTW, KTL, &fused_fwd_kernel<CELL_LSTM, false, false, NCW, KS, MTW, KTW, KTL>},
const FusedVariant kTable[] = {FRNN_FUSED_DESIGNS(FRNN_FV) FRNN_FUSED_RLDS_DESIGNS(FRNN_FVL)};
#undef FRNN_FV
#undef FRNN_FVL

#define FRNN_FBV(NCW, KS, MTW, KTW) \
  {CELL_LSTM, NCW, KS, MTW, KTW, &fused_bwd_kernel<CELL_LSTM, NCW, KS, MTW, KTW>},
const FusedBwdVariant kBwdTable[] = {FRNN_FUSED_BWD_LSTM(FRNN_FBV)};
#undef FRNN_FBV

#define FRNN_FBXV(NCW, MTW, KTW) \
  {CELL_LSTM, NCW, MTW, KTW, 0, &fused_bwdx_kernel<CELL_LSTM, NCW, MTW, KTW>},
#define FRNN_FBXVL(NCW, MTW, KTW, KTL) \
  {CELL_LSTM, NCW, MTW, KTW, KTL, &fused_bwdx_kernel<CELL_LSTM, NCW, MTW, KTW, KTL>},
const FusedBwdxVariant kBwdxTable[] = {FRNN_FUSED_BWDX_LSTM(FRNN_FBXV) FRNN_FUSED_BWDX_RLDS_LSTM(FRNN_FBXVL)};
#undef FRNN_FBXV
#undef FRNN_FBXVL

}  // namespace

FusedBwdxTable fused_bwdx_table_lstm() {
  return FusedBwdxTable{kBwdxTable, (int)(sizeof(kBwdxTable) / sizeof(kBwdxTable[0]))};
}

FusedBwdTable fused_bwd_table_lstm() { return FusedBwdTable{kBwdTable, (int)(sizeof(kBwdTable) / sizeof(kBwdTable[0]))}; }

fused_bwd_fn fused_bwd_local_lstm(int D, bool bf) {
  if (D == 32) return bf ? &fused_bwd_local_kernel<CELL_LSTM, 4 * 32 / 32, true> : &fused_bwd_local_kernel<CELL_LSTM, 4 * 32 / 4, false>;
  if (D == 64) return bf ? &fused_bwd_local_kernel<CELL_LSTM, 4 * 64 / 32, true> : &fused_bwd_local_kernel<CELL_LSTM, 4 * 64 / 4, false>;
  return nullptr;
}

FusedTable fused_table_lstm() { return FusedTable{kTable, (int)(sizeof(kTable) / sizeof(kTable[0]))}; }

}  // namespace frnn
