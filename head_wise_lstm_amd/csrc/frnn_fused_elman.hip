// Instantiations of the fused forward and backward kernels for the elman cell (one translation
// unit per cell).
#include "frnn_variants.hpp"

namespace frnn {
namespace {

#define FRNN_FV(F32, LOCAL, NCW, KS, MTW, KTW) \
  {CELL_ELMAN, F32, LOCAL, NCW, KS, MTW, KTW, 0, &fused_fwd_kernel<CELL_ELMAN, F32, LOCAL, NCW, KS, MTW, KTW>},
const FusedVariant kTable[] = {FRNN_FUSED_DESIGNS(FRNN_FV)};
#undef FRNN_FV

#define FRNN_FBV(NCW, KS, MTW, KTW) \
  {CELL_ELMAN, NCW, KS, MTW, KTW, &fused_bwd_kernel<CELL_ELMAN, NCW, KS, MTW, KTW>},
const FusedBwdVariant kBwdTable[] = {FRNN_FUSED_BWD_ELMAN(FRNN_FBV)};
#undef FRNN_FBV

#define FRNN_FBXV(NCW, MTW, KTW) \
  {CELL_ELMAN, NCW, MTW, KTW, 0, &fused_bwdx_kernel<CELL_ELMAN, NCW, MTW, KTW>},
const FusedBwdxVariant kBwdxTable[] = {FRNN_FUSED_BWDX_ELMAN(FRNN_FBXV)};
#undef FRNN_FBXV

}  // namespace

FusedBwdxTable fused_bwdx_table_elman() {
  return FusedBwdxTable{kBwdxTable, (int)(sizeof(kBwdxTable) / sizeof(kBwdxTable[0]))};
}

FusedBwdTable fused_bwd_table_elman() { return FusedBwdTable{kBwdTable, (int)(sizeof(kBwdTable) / sizeof(kBwdTable[0]))}; }

fused_bwd_fn fused_bwd_local_elman(int D, bool bf) {
  if (D == 32) return bf ? &fused_bwd_local_kernel<CELL_ELMAN, 1 * 32 / 32, true> : &fused_bwd_local_kernel<CELL_ELMAN, 1 * 32 / 4, false>;
  if (D == 64) return bf ? &fused_bwd_local_kernel<CELL_ELMAN, 1 * 64 / 32, true> : &fused_bwd_local_kernel<CELL_ELMAN, 1 * 64 / 4, false>;
  return nullptr;
}

FusedTable fused_table_elman() { return FusedTable{kTable, (int)(sizeof(kTable) / sizeof(kTable[0]))}; }

}  // namespace frnn
