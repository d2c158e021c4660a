// Instantiations of the fused kernel for the gru cell (one translation unit per cell).
#include "frnn_variants.hpp"

namespace frnn {
namespace {

#define FRNN_FV(F32, LOCAL, NCW, KS, MTW, KTW) \
  {CELL_GRU, F32, LOCAL, NCW, KS, MTW, KTW, &fused_fwd_kernel<CELL_GRU, F32, LOCAL, NCW, KS, MTW, KTW>},
const FusedVariant kTable[] = {FRNN_FUSED_DESIGNS(FRNN_FV)};
#undef FRNN_FV

}  // namespace

FusedTable fused_table_gru() { return FusedTable{kTable, (int)(sizeof(kTable) / sizeof(kTable[0]))}; }

}  // namespace frnn
