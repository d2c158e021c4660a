// Host side of libfrnn: argument validation, launch planning, workspace layout and the C ABI
// declared in include/frnn.h. Validation and planning are plain host code and run before any HIP
// call, so they are testable without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "frnn.h"
#include "frnn_alt.hpp"
#include "frnn_bwd.hpp"
#include "frnn_device.hpp"
#include "frnn_proj.hpp"
#include "frnn_rpack.hpp"
#include "frnn_variants.hpp"

using namespace frnn;

namespace {

// ----------------------------------------------------------------------------- small kernels
__global__ void __launch_bounds__(256) fill_u32_kernel(uint32_t* p, long long n, uint32_t v) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) p[i] = v;
}

// last_states <- states0 (or zeros) for T == 0, widened to fp32. n = S * B * N * D elements.
__global__ void __launch_bounds__(256) copy_init_kernel(const void* s0, int s0_f32, float* dst, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
    dst[i] = s0 ? ld_f(s0, i, s0_f32) : 0.0f;
}

// dst[r][c] = src[r][c] for r < rows, c < cols (bf16, row strides sld and dld elements): places
// one matrix beside another, e.g. two directions' Wi side by side along K.
__global__ void __launch_bounds__(256) copy_rows_b16_kernel(const uint16_t* src, long long sld, int rows, int cols,
                                                            uint16_t* dst, long long dld) {
  const long long n = (long long)rows * cols;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const long long r = i / cols, c = i - r * cols;
    dst[r * dld + c] = src[r * sld + c];
  }
}

// Both biases of a bidirectional layer in the projection's column order [gate][direction][unit]:
// out[j] from b_ih, out[4*dirs*H + j] from b_hh (bf16, a NULL bias reads as zeros).
struct StackBiasArgs {
  int H, dirs;
  const uint16_t* bi[2];
  const uint16_t* bh[2];
  uint16_t* out;
};

__global__ void __launch_bounds__(256) stack_bias_kernel(StackBiasArgs a) {
  const int G4 = 4 * a.H * a.dirs;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= G4) return;
  const int g = j / (a.dirs * a.H), r = j - g * a.dirs * a.H, n = r / a.H, e = r - n * a.H;
  const int src = g * a.H + e;
  a.out[j] = a.bi[n] ? a.bi[n][src] : (uint16_t)0;
  a.out[G4 + j] = a.bh[n] ? a.bh[n][src] : (uint16_t)0;
}

// Records the hardware die id of each workgroup (used once to learn the dispatch pattern).
__global__ void xcc_map_kernel(int* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = xcc_id();
}

constexpr size_t kErrBytes = 256;
constexpr int kMaxDies = 8;
constexpr size_t kCtrBytes = 256;  // per-die workgroup counters after a launch's exchange words

// The workspace of frnn_fwd_noalloc: one array per device, held until the process ends. Host code
// never uses this name as an address (on the host it is a stand-in); init_device() looks up the
// device address of the current device's copy once and every use goes through that pointer.
constexpr size_t kScratchBytes = FRNN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ----------------------------------------------------------------------------- device facts
struct DevInfo {
  bool ok = false;
  int device = -1;
  int cus = 256;
  int n_xcd = 8;
  bool periodic = true;
  int xcc_of[kMaxDies] = {0, 1, 2, 3, 4, 5, 6, 7};
  long long wall_khz = 100000;
  void* scratch = nullptr;  // device address of this device's `scratch` array
};

std::mutex g_dev_mu;
std::vector<DevInfo> g_dev;

int raise_lds_limits();

// Learns the facts of the current device once (frnn_init): its architecture, CU count and wall
// clock, and how workgroups are dealt to dies: a grid of one workgroup per CU records the die id
// of each. The fused designs need the pattern to be periodic in the workgroup index.
int init_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FRNN_ENODEVICE;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if ((int)g_dev.size() <= dev) g_dev.resize(dev + 1);
  DevInfo& di = g_dev[dev];
  if (di.ok) return FRNN_OK;
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) return FRNN_ENODEVICE;
  if (std::strncmp(p.gcnArchName, "gfx950", 6) != 0) return FRNN_ENODEVICE;
  DevInfo nd;
  nd.device = dev;
  nd.cus = p.multiProcessorCount;
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess && khz > 0) nd.wall_khz = khz;
  nd.n_xcd = std::max(1, std::min(kMaxDies, nd.cus / 32));
  const int nb = nd.cus;
  int* d_map = nullptr;
  std::vector<int> map(nb, -1);
  if (hipMalloc(&d_map, sizeof(int) * nb) != hipSuccess) return FRNN_EHIP;
  hipLaunchKernelGGL(xcc_map_kernel, dim3(nb), dim3(64), 0, 0, d_map);
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(map.data(), d_map, sizeof(int) * nb, hipMemcpyDeviceToHost);
  (void)hipFree(d_map);
  if (e != hipSuccess) return FRNN_EHIP;
  nd.periodic = true;
  for (int d = 0; d < nd.n_xcd; ++d) nd.xcc_of[d] = map[d];
  for (int b = 0; b < nb; ++b)
    if (map[b] != map[b % nd.n_xcd]) nd.periodic = false;
  for (int d = 0; d < nd.n_xcd; ++d)
    for (int d2 = 0; d2 < d; ++d2)
      if (nd.xcc_of[d] == nd.xcc_of[d2]) nd.periodic = false;
  const int rc = raise_lds_limits();
  if (rc != FRNN_OK) return rc;
  if (hipGetSymbolAddress(&nd.scratch, HIP_SYMBOL(scratch)) != hipSuccess || !nd.scratch) return FRNN_EHIP;
  nd.ok = true;
  di = nd;
  return FRNN_OK;
}

// The facts frnn_init() learned for the current device (a host-side lookup: no device call
// beyond asking which device is current).
int get_devinfo(DevInfo* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FRNN_ENODEVICE;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if ((int)g_dev.size() <= dev || !g_dev[dev].ok) return FRNN_ENOINIT;
  *out = g_dev[dev];
  return FRNN_OK;
}

DevInfo default_devinfo() { return DevInfo(); }

// Launch of a persistent kernel whose workgroups wait on each other (bounded waits): every
// workgroup must be resident at once. The planner keeps the grid within one workgroup per CU; this
// checks on the host that the kernel's registers and LDS allow that many (hipOccupancy is a host
// query), then makes a plain launch. The hardware deals workgroups to dies round-robin in a plain
// launch too (the probe of init_device is one). A cooperative launch is not used: nothing here
// needs its grid-wide barrier, and every profiled process that made one ended in a segmentation
// fault inside exit(), after the profiler's own teardown, while processes with plain launches only
// exited normally.
int launch_resident(const void* fn, int grid, int threads, size_t lds, void** args, int cus, hipStream_t st) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) != hipSuccess) return FRNN_EHIP;
  if ((long long)per_cu * cus < grid) return FRNN_ENORESIDENT;
  return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, lds, st) == hipSuccess ? FRNN_OK : FRNN_EHIP;
}

// ----------------------------------------------------------------------------- kernel tables
// The instantiated design with these variables and R^T wholly in VGPRs (ktl = 0), or, with
// ktl < 0, the one that keeps the fewest k-tiles of it in LDS.
const FusedVariant* find_fused(int cell, int f32, int local, int ncw, int ks, int mtw, int ktw, int ktl = 0) {
  const FusedTable t = cell == FRNN_CELL_LSTM ? fused_table_lstm()
                       : cell == FRNN_CELL_GRU ? fused_table_gru()
                                               : fused_table_elman();
  const FusedVariant* best = nullptr;
  for (int i = 0; i < t.n; ++i) {
    const FusedVariant& v = t.v[i];
    if (v.cell != cell || v.f32 != f32 || v.local != local || v.ncw != ncw || v.ks != ks || v.mtw != mtw ||
        v.ktw != ktw)
      continue;
    if (ktl >= 0 ? v.ktl == ktl : (v.ktl > 0 && (!best || v.ktl < best->ktl))) {
      if (ktl >= 0) return &v;
      best = &v;
    }
  }
  return best;
}

const FusedBwdVariant* find_fused_bwd(int cell, int ncw, int ks, int mtw, int ktw) {
  const FusedBwdTable t = cell == FRNN_CELL_LSTM ? fused_bwd_table_lstm()
                          : cell == FRNN_CELL_GRU ? fused_bwd_table_gru()
                                                  : fused_bwd_table_elman();
  for (int i = 0; i < t.n; ++i) {
    const FusedBwdVariant& v = t.v[i];
    if (v.cell == cell && v.ncw == ncw && v.ks == ks && v.mtw == mtw && v.ktw == ktw) return &v;
  }
  return nullptr;
}

// ktl < 0: the design with the fewest k-tiles of R in LDS.
const FusedBwdxVariant* find_fused_bwdx(int cell, int ncw, int mtw, int ktw, int ktl = -1) {
  const FusedBwdxTable t = cell == FRNN_CELL_LSTM ? fused_bwdx_table_lstm()
                           : cell == FRNN_CELL_GRU ? fused_bwdx_table_gru()
                                                   : fused_bwdx_table_elman();
  const FusedBwdxVariant* best = nullptr;
  for (int i = 0; i < t.n; ++i) {
    const FusedBwdxVariant& v = t.v[i];
    if (v.cell != cell || v.ncw != ncw || v.mtw != mtw || v.ktw != ktw) continue;
    if (ktl >= 0 ? v.ktl == ktl : (!best || v.ktl < best->ktl)) {
      if (ktl >= 0) return &v;
      best = &v;
    }
  }
  return best;
}

// Raises the dynamic-LDS limit of every persistent kernel to what its design uses (frnn_init), so
// that a compute call makes no attribute call. A design's head width is fixed by its k-tiles, so
// its LDS is known here exactly as the planner computes it.
constexpr int kMaxLds = 160 * 1024;

int raise_lds_limits() {
  auto raise = [](const void* fn, int bytes) {
    if (bytes <= 48 * 1024) return true;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, std::min(bytes, kMaxLds)) == hipSuccess;
  };
  for (const FusedTable& t : {fused_table_lstm(), fused_table_elman(), fused_table_gru()}) {
    for (int i = 0; i < t.n; ++i) {
      const FusedVariant& v = t.v[i];
      const int D = v.ks * v.ktw * (v.f32 ? 4 : 32);
      if (!raise(reinterpret_cast<const void*>(v.fn), fused_lds(v.local, v.f32, v.ncw, v.ks, v.mtw, D, v.cell, v.ktl).total))
        return FRNN_EHIP;
    }
  }
  for (const FusedBwdTable& t : {fused_bwd_table_lstm(), fused_bwd_table_elman(), fused_bwd_table_gru()}) {
    for (int i = 0; i < t.n; ++i) {
      const FusedBwdVariant& v = t.v[i];
      const int U = (v.ncw / v.ks) * v.mtw * 16;
      if (!raise(reinterpret_cast<const void*>(v.fn), fused_bwd_lds(v.ncw, v.ks, v.mtw, v.ktw, FUSED_DIE_MAX_BR, U).total))
        return FRNN_EHIP;
    }
  }
  for (const FusedBwdxTable& t : {fused_bwdx_table_lstm(), fused_bwdx_table_elman(), fused_bwdx_table_gru()}) {
    for (int i = 0; i < t.n; ++i) {
      const FusedBwdxVariant& v = t.v[i];
      const int UW = v.ktw * 32 / cell_gates(v.cell);
      if (!raise(reinterpret_cast<const void*>(v.fn), fused_bwdx_lds(v.ktw, FUSED_DIE_MAX_BR, UW, v.ncw, v.mtw, v.ktl).total))
        return FRNN_EHIP;
    }
  }
  for (const int D : {32, 64}) {
    for (const bool bf : {false, true}) {
      const fused_bwd_fn fns[3] = {fused_bwd_local_lstm(D, bf), fused_bwd_local_gru(D, bf), fused_bwd_local_elman(D, bf)};
      const int gates[3] = {4, 3, 1};
      for (int c = 0; c < 3; ++c)
        if (fns[c] && !raise(reinterpret_cast<const void*>(fns[c]), fused_bwdl_lds(gates[c], D, fused_bwdl_max_br(D), bf).total))
          return FRNN_EHIP;
    }
  }
  return FRNN_OK;
}

// ----------------------------------------------------------------------------- problem
struct Problem {
  int B, T, N, D, cell;
  int r_f32;   // R / bias / MFMA operand type fp32 (else bf16)
  const void* Wx;
  int wx_f32;
  long long wx_sb, wx_st;
  const void* R;
  long long r_sg, r_sn, r_sd;
  const void* bias;
  const void* s0_h;
  const void* s0_c;
  int s0_f32;
  long long s0_sb, s0_sn;
  float* out_h;
  float* out_c;
  long long out_sb, out_st;
  float* last_h;
  float* last_c;
  long long last_sb, last_sn;
  int rev_n0;  // heads n >= rev_n0 run backwards in time (N: none)
};

// Gates stored in Wx, R and b; rows per unit in a tile of packed R^T (see cell_slots).
int gates_of(int cell) { return cell_gates(cell); }
int slots_of(int cell) { return cell_slots(cell); }
const char* cell_name(int cell) { return cell == FRNN_CELL_LSTM ? "lstm" : cell == FRNN_CELL_GRU ? "gru" : "elman"; }

struct FusedPlan {
  const FusedVariant* v = nullptr;
  int local = 0, W = 1, BR = 16, groups = 0, ncw = 4, ks = 1, mtw = 0, ktw = 0, n_xcd = 1, slots = 0, grid = 0;
  int ktl = 0;             // k-tiles per compute wave whose R^T fragments live in LDS
  int chunks = 1, Bc = 0;  // the batch runs as `chunks` launches of at most Bc rows
  double cost_us = 0.0;    // predicted time of the whole call
  size_t lds = 0;
};

int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  if (!s || !*s) return dflt;
  return std::atoi(s);
}

// Predicted time of one step of the fused kernel (µs). Die-local design: fitted by least squares
// to 129 measured die-local designs on twelve shapes (LSTM, GRU, Elman; D 64-768; B 4-64; the
// kernels with 16-byte exchange polls): a base for the exchange, the barrier and the gates, plus
// each compute wave's MFMA chain (MTW*KTW tiles), its poll loads per lane and round, and the
// number of compute waves (more waves meet at every barrier and split the K-sum exchange). The
// single-workgroup design has no exchange; its chain runs over the whole K. Fitted by least squares
// to 110 measured single-workgroup designs on thirteen shapes (LSTM, GRU, Elman; D 32-128; B
// 16-128; N 2-12; RMS 33 ns): a base per cell (what the I/O wave streams and the gates cost: the
// LSTM's four gates of Wx, five transcendentals and two states a unit, the GRU's three, three and
// one, the Elman head's one gate through its DMA ring), the MFMA chain, and two batch-row terms:
// one growing with the rows (the states the compute waves store, the Wx words the I/O wave loads)
// and one falling with them, fitted to the measurement that one row a workgroup runs slower than
// two to four on every swept shape (with a row term alone the model picked one row and lost up to
// 7 % against the best design; with both, its worst pick over 28 shapes loses 4.4 %).
constexpr double kStepBaseDie = 0.700, kStepPerMfma = 0.0164, kStepPerPollLoad = 0.0141, kStepPerWave = 0.0181;
constexpr double kStepBaseLocalLstm = 0.356, kStepBaseLocalGru = 0.157, kStepBaseLocalElman = 0.075;
constexpr double kStepPerMfmaLocal = 0.0495, kStepPerRowLocal = 0.0193, kStepPerInvRowLocal = 0.079;
// A die-local design with part of R^T in LDS reads MTW*KTL fragments (1 KB each) from LDS per wave
// and step, the CU's eight compute waves sharing the LDS port: its step adds this per fragment.
constexpr double kStepPerRLds = 0.027;
constexpr double kLaunchUs = 15.0;  // R packing, fills and the launch of one chunk

double step_cost(bool local, int cell, int br, int ncw, int ks, int mtw, int ktw, int ktl = 0) {
  if (local) {
    const double base = cell == FRNN_CELL_LSTM ? kStepBaseLocalLstm : cell == FRNN_CELL_GRU ? kStepBaseLocalGru
                                                                                           : kStepBaseLocalElman;
    return base + kStepPerMfmaLocal * mtw * ktw + kStepPerRowLocal * br + kStepPerInvRowLocal / br;
  }
  const int np = (br * ktw * 32 / fused_poll_words(ks, mtw, ktw) + 63) / 64;
  return kStepBaseDie + kStepPerMfma * mtw * ktw + kStepPerPollLoad * np + kStepPerWave * ncw + kStepPerRLds * mtw * ktl;
}

// Choose the fused design by integer constraint search. The variables are:
//   single-workgroup or die-local; batch rows per group BR; workgroups per group W;
//   compute waves and K split (NCW, KS), which fix the tiles and k-tiles per wave (MTW, KTW);
//   and the number of batch chunks.
// The constraints are:
//   divisibility of the head's tiles and k-tiles;
//   an instantiated kernel for the design (each fits the register file without spilling);
//   the K-split packing's and the I/O wave's batch-row limits;
//   co-residency: one workgroup per CU, a group's workgroups on one die.
// The objective is the predicted time of the call: chunks x (T x step cost + launch). A batch
// that cannot be co-resident runs as several launches over chunks of rows (rows never interact).
// FRNN_FUSED_W / BR / NCW / KS pin variables for measurements.
int plan_fused(const Problem& p, const DevInfo& di, FusedPlan* out) {
  const int G = gates_of(p.cell);
  const int GS = slots_of(p.cell);
  const int TPH = GS * p.D / 16;
  const int KW = p.r_f32 ? 4 : 32;
  if (p.D % 32 != 0 || TPH < 1) return FRNN_EUNSUPPORTED;
  const int KT = p.D / KW;
  const int force_w = env_int("FRNN_FUSED_W", 0);
  const int force_br = env_int("FRNN_FUSED_BR", 0);
  const int force_ncw = env_int("FRNN_FUSED_NCW", 0), force_ks = env_int("FRNN_FUSED_KS", 0);
  const int T = std::max(p.T, 1);
  FusedPlan best;
  bool found = false;
  auto consider = [&](FusedPlan fp, int max_groups) {
    // the largest chunk of rows whose groups fit at once, and the chunks the batch needs
    if (max_groups < p.N) return;
    const long long bmax = (long long)fp.BR * (max_groups / p.N);
    fp.chunks = (int)((p.B + bmax - 1) / bmax);
    fp.Bc = (int)(((long long)p.B + fp.chunks - 1) / fp.chunks);
    fp.groups = p.N * ((fp.Bc + fp.BR - 1) / fp.BR);
    fp.cost_us = fp.chunks * (T * step_cost(fp.local, p.cell, fp.BR, fp.ncw, fp.ks, fp.mtw, fp.ktw, fp.ktl) + kLaunchUs);
    if (!fp.local) {
      const int per_die = (fp.groups + di.n_xcd - 1) / di.n_xcd;
      fp.slots = per_die * fp.W;
      fp.grid = fp.slots * di.n_xcd;
    } else {
      fp.grid = fp.groups;
    }
    // ties: fewer chunks, then fewer rows per group
    if (!found || fp.cost_us < best.cost_us - 1e-9 ||
        (std::abs(fp.cost_us - best.cost_us) <= 1e-9 && (fp.chunks < best.chunks || (fp.chunks == best.chunks && fp.BR < best.BR)))) {
      best = fp;
      found = true;
    }
  };
  // single-workgroup design: a whole head per workgroup, one workgroup per CU
  if (force_w <= 1 && !force_ks) {
    for (int ncw : {4, 8}) {
      if (force_ncw && ncw != force_ncw) continue;
      const int mtw = (TPH + ncw - 1) / ncw;
      const FusedVariant* v = find_fused(p.cell, p.r_f32, 1, ncw, 1, mtw, KT);
      if (!v) continue;
      // a long per-wave MFMA chain makes the die-local split faster (measured); keep the design
      // for heads whose chain is short
      if (mtw * KT > 64 && force_w != 1) continue;
      // the I/O wave moves at most 64 * epl words of Wx per step (the compute waves store the
      // states themselves in this design)
      const int epl = fused_epl(true, ncw, p.cell, 1, mtw);
      const int words_per_row = G * p.D / (p.wx_f32 ? 2 : 4);
      const int br_cap = std::min(16, 64 * epl / words_per_row);
      for (int br = 1; br <= br_cap; ++br) {
        if (force_br && br != force_br) continue;
        FusedPlan fp;
        fp.v = v; fp.local = 1; fp.W = 1; fp.BR = br; fp.ncw = ncw; fp.ks = 1; fp.mtw = mtw; fp.ktw = KT;
        fp.lds = (size_t)fused_lds(true, p.r_f32, ncw, 1, mtw, p.D, p.cell).total;
        consider(fp, di.cus);
      }
    }
  }
  // die-local design: W workgroups per group on one die
  if (!p.r_f32 && di.periodic && force_w != 1) {
    const int slots_per_die = std::max(1, di.cus / di.n_xcd);
    const int cand[][2] = {{4, 1}, {4, 2}, {4, 4}, {6, 6}, {8, 2}, {8, 4}, {8, 8}};
    for (int BR = 1; BR <= FUSED_DIE_MAX_BR; ++BR) {
      if (force_br && BR != force_br) continue;
      for (int W = 2; W <= std::min(32, slots_per_die); ++W) {
        if ((force_w > 1 && W != force_w) || TPH % W) continue;
        const int mt_wg = TPH / W;
        const int u_wg = mt_wg * (GS == 4 ? 4 : 16);
        for (const auto& nk : cand) {
          const int ncw = nk[0], ks = nk[1];
          if ((force_ncw && ncw != force_ncw) || (force_ks && ks != force_ks)) continue;
          const int ms = ncw / ks;
          if (mt_wg % ms || KT % ks) continue;
          const int mtw = mt_wg / ms, ktw = KT / ks;
          // R^T wholly in registers where a design holds it, else in part in LDS
          const FusedVariant* v = find_fused(p.cell, 0, 0, ncw, ks, mtw, ktw);
          if (!v) v = find_fused(p.cell, 0, 0, ncw, ks, mtw, ktw, -1);
          if (!v || BR > fused_max_br(ks, mtw)) continue;
          // the I/O wave moves at most 64 * epl words of Wx and as many output pairs per step
          const int epl = fused_epl(false, ncw, p.cell, ks, mtw);
          if (BR * G * u_wg / (p.wx_f32 ? 2 : 4) > 64 * epl || BR * u_wg / 2 > 64 * epl) continue;
          FusedPlan fp;
          fp.v = v; fp.local = 0; fp.W = W; fp.BR = BR; fp.ncw = ncw; fp.ks = ks; fp.mtw = mtw; fp.ktw = ktw;
          fp.n_xcd = di.n_xcd;
          fp.ktl = v->ktl;
          fp.lds = (size_t)fused_lds(false, false, ncw, ks, mtw, p.D, p.cell, v->ktl).total;
          if (fp.lds > (size_t)kMaxLds) continue;
          consider(fp, (slots_per_die / W) * di.n_xcd);
        }
      }
    }
  }
  if (!found) return FRNN_EUNSUPPORTED;
  *out = best;
  return FRNN_OK;
}

// Scratch needed by the recurrence of a problem on a path, beside the error word (independent
// of T).
size_t rec_scratch_bytes(int B, int N, int D, int cell, int r_f32, int path) {
  const int GS = slots_of(cell);
  const size_t elt = r_f32 ? 4 : 2;
  size_t s = align256((size_t)GS * N * D * D * elt);  // packed R
  if (path == FRNN_PATH_FUSED) {
    // exchange words: groups * BR <= N * (B + 15) rows, two parities; the per-die counters
    return s + align256((size_t)2 * N * (B + 15) * D * 4) + kCtrBytes;
  }
  s += 2 * align256((size_t)N * B * D * elt);  // h, two buffers
  s += align256((size_t)B * N * D * 4);        // current c
  return s;
}

// R^T into MFMA fragment order (rpack); the coalesced kernel when the strides allow 8-byte rows.
hipError_t launch_rpack(const Problem& p, void* out, hipStream_t st) {
  RpackArgs ra;
  ra.N = p.N; ra.D = p.D; ra.cell = p.cell; ra.R = p.R;
  ra.r_sg = p.r_sg; ra.r_sn = p.r_sn; ra.r_sd = p.r_sd; ra.out = out;
  const bool vec = !p.r_f32 && p.D % 32 == 0 && ((p.r_sg | p.r_sn | p.r_sd) & 3) == 0 &&
                   (reinterpret_cast<uintptr_t>(p.R) & 7u) == 0;
  if (vec) {
    hipLaunchKernelGGL(rpack_bf16_kernel, dim3((p.D + RPACK_UB - 1) / RPACK_UB, p.D / 32, p.N), dim3(256), 0, st, ra);
  } else {
    const long long total = (long long)p.N * (slots_of(p.cell) * p.D / 16) * (p.D / (p.r_f32 ? 4 : 32)) * 64;
    hipLaunchKernelGGL(rpack_any_kernel, dim3((unsigned)std::min<long long>((total + 255) / 256, 4096)), dim3(256), 0,
                       st, ra, p.r_f32);
  }
  return hipGetLastError();
}

hipError_t launch_fill(void* p, size_t bytes, hipStream_t st, uint32_t value = 0u) {
  const long long n = (long long)(bytes / 4);
  if (n <= 0) return hipSuccess;
  const int blocks = (int)std::min<long long>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks), dim3(256), 0, st, reinterpret_cast<uint32_t*>(p), n, value);
  return hipGetLastError();
}

// dst[j][k] = src[k][j] (K rows of Nc elements, 2- or 4-byte elements), for mats matrices in one
// launch, matrix z at src + z * src_z and dst + z * dst_z.
template <typename E>
void launch_transpose(const E* src, long long lds, int K, int Nc, E* dst, long long ldd, hipStream_t st, int mats = 1,
                      long long src_z = 0, long long dst_z = 0) {
  if (K <= 0 || Nc <= 0 || mats <= 0) return;
  if (sizeof(E) == 2 && lds % 4 == 0 && ldd % 4 == 0 && src_z % 4 == 0 && dst_z % 4 == 0 &&
      !(reinterpret_cast<uintptr_t>(src) & 7) && !(reinterpret_cast<uintptr_t>(dst) & 7)) {
    const int ty = (int)std::min<long long>(((long long)K + 63) / 64, 65535);
    hipLaunchKernelGGL(transpose_b16_kernel, dim3((Nc + 63) / 64, ty, mats), dim3(256), 0, st,
                       reinterpret_cast<const uint16_t*>(src), lds, K, Nc, reinterpret_cast<uint16_t*>(dst), ldd, src_z,
                       dst_z);
    return;
  }
  const int ty = (int)std::min<long long>(((long long)K + 31) / 32, 65535);
  hipLaunchKernelGGL(transpose_kernel<E>, dim3((Nc + 31) / 32, ty, mats), dim3(256), 0, st, src, lds, K, Nc, dst, ldd,
                     src_z, dst_z);
}

// Launch of the bf16 GEMM of ProjArgs: with bf16 A whose rows (and Bt's, and the parts' offsets)
// start on 16-byte boundaries, the kernel that loads its tiles straight into LDS (128-row tiles
// where the product has at most 128 rows); otherwise the register-staged one (fp32 A is rounded
// as it is staged). FRNN_PROJ_DMA=0 pins the latter. The grid's x is proj_tiles(pa).
bool proj_dma(const ProjArgs& pa) {
  const bool aligned = reinterpret_cast<uintptr_t>(pa.A) % 16 == 0 && reinterpret_cast<uintptr_t>(pa.Bt) % 16 == 0 &&
                       pa.lda % 8 == 0 && pa.ldb % 8 == 0 && pa.a_z % 8 == 0 && pa.b_z % 8 == 0 &&
                       pa.a_h % 8 == 0 && pa.b_h % 8 == 0;
  return !pa.a_f32 && aligned && env_int("FRNN_PROJ_DMA", 1);
}
int proj_bm(const ProjArgs& pa) { return proj_dma(pa) && pa.M <= 128 ? 128 : PJ_BM; }
unsigned proj_tiles(const ProjArgs& pa) {
  const int bm = proj_bm(pa);
  return (unsigned)(((pa.Nc + PJ_BN - 1) / PJ_BN) * ((pa.M + bm - 1) / bm));
}

void launch_proj(const ProjArgs& pa, dim3 grid, hipStream_t st) {
  if (pa.M <= 0 || pa.Nc <= 0) return;
  const bool dma = proj_dma(pa), small = proj_bm(pa) == 128;
  if (pa.nt) {
    if (pa.a_f32) hipLaunchKernelGGL((proj_gemm_kernel<true, true>), grid, dim3(256), 0, st, pa);
    else if (dma && small) hipLaunchKernelGGL((proj_gemm_dma_kernel<true, 128>), grid, dim3(256), 0, st, pa);
    else if (dma) hipLaunchKernelGGL((proj_gemm_dma_kernel<true>), grid, dim3(256), 0, st, pa);
    else hipLaunchKernelGGL((proj_gemm_kernel<false, true>), grid, dim3(256), 0, st, pa);
  } else {
    if (pa.a_f32) hipLaunchKernelGGL((proj_gemm_kernel<true, false>), grid, dim3(256), 0, st, pa);
    else if (dma && small) hipLaunchKernelGGL((proj_gemm_dma_kernel<false, 128>), grid, dim3(256), 0, st, pa);
    else if (dma) hipLaunchKernelGGL((proj_gemm_dma_kernel<false>), grid, dim3(256), 0, st, pa);
    else hipLaunchKernelGGL((proj_gemm_kernel<false, false>), grid, dim3(256), 0, st, pa);
  }
}

// C[M][Nc] = A[M][K] . Bt[Nc][K]^T in fp32, for parts y = 0 .. parts-1 of heads z = 0 .. heads-1
// at once (A, Bt and C offset by y * a_z + z * a_h, y * b_z + z * b_h, y * c_z + z * c_h
// elements): the tiled MFMA kernel for bf16 operands, the plain fp32 MFMA kernel for fp32 ones. K
// is a multiple of 32.
hipError_t launch_gemm(bool f32, int M, int Nc, int K, const void* A, long long lda, const void* Bt, long long ldb,
                       float* C, long long ldc, hipStream_t st, int parts = 1, long long a_z = 0, long long b_z = 0,
                       long long c_z = 0, bool a_f32 = false, int heads = 1, long long a_h = 0, long long b_h = 0,
                       long long c_h = 0) {
  if (M <= 0 || Nc <= 0) return hipSuccess;
  if (K % 32 != 0 || parts < 1 || heads < 1 || heads > 65535) return hipErrorInvalidValue;
  if (f32) {
    const long long tiles = (long long)((M + 15) / 16) * ((Nc + 15) / 16);
    hipLaunchKernelGGL(gemm_f32_kernel, dim3((unsigned)((tiles + 3) / 4), parts, heads), dim3(256), 0, st, M, Nc, K,
                       reinterpret_cast<const float*>(A), lda, reinterpret_cast<const float*>(Bt), ldb, C, ldc, a_z, b_z,
                       c_z, a_h, b_h, c_h);
    return hipGetLastError();
  }
  ProjArgs pa;
  pa.M = M; pa.Nc = Nc; pa.K = K;
  pa.A = A; pa.a_f32 = a_f32 ? 1 : 0; pa.lda = lda;
  pa.Bt = reinterpret_cast<const uint16_t*>(Bt);
  pa.ldb = ldb;
  pa.b1 = nullptr; pa.b2 = nullptr;
  pa.C = C; pa.ldc = ldc;
  pa.a_z = a_z; pa.b_z = b_z; pa.c_z = c_z;
  pa.a_h = a_h; pa.b_h = b_h; pa.c_h = c_h;
  pa.nt = 1;  // every caller's product is read by a streaming kernel
  const dim3 pgrid(proj_tiles(pa), parts, heads);
  launch_proj(pa, pgrid, st);
  return hipGetLastError();
}

void trace(const char* fmt, const std::string& s) {
  if (env_int("FRNN_TRACE", 0)) std::fprintf(stderr, fmt, s.c_str());
}

std::string plan_string(const Problem& p, int path, const FusedPlan* fp) {
  char buf[512];
  if (path == FRNN_PATH_FUSED && fp) {
    std::snprintf(buf, sizeof(buf),
                  "fused design=%s cell=%s dtype=%s B=%d T=%d N=%d D=%d BR=%d groups=%d W=%d NCW=%d KS=%d MTW=%d KTW=%d%s "
                  "dies=%d slots/die=%d grid=%d lds=%zu chunks=%d rows/chunk=%d predicted_us=%.1f",
                  fp->local ? "workgroup-local" : "die-local", cell_name(p.cell),
                  p.r_f32 ? "f32" : "bf16", p.B, p.T, p.N, p.D, fp->BR, fp->groups, fp->W, fp->ncw, fp->ks, fp->mtw, fp->ktw,
                  fp->ktl > 0 ? (" KTL=" + std::to_string(fp->ktl)).c_str() : "", fp->n_xcd, fp->slots, fp->grid, fp->lds,
                  fp->chunks, fp->Bc, fp->cost_us);
  } else {
    const int TPH = slots_of(p.cell) * p.D / 16;
    std::snprintf(buf, sizeof(buf),
                  "alternating cell=%s dtype=%s B=%d T=%d N=%d D=%d step_grid=(%d,%d,%d) launches=%d",
                  cell_name(p.cell), p.r_f32 ? "f32" : "bf16", p.B, p.T, p.N, p.D,
                  TPH, (p.B + 15) / 16, p.N, p.T + 2);
  }
  return std::string(buf);
}

// Run the recurrence of a validated problem. `scratch` holds at least rec_scratch_bytes();
// device-side errors are or-ed into `err` (cleared by the caller once per API call).
int run_recurrence(const Problem& p, int path, int* err, void* scratch, hipStream_t st) {
  DevInfo di;
  int rc = get_devinfo(&di);
  if (rc != FRNN_OK) return rc;
  char* base = reinterpret_cast<char*>(scratch);
  if (path == FRNN_PATH_FUSED) {
    FusedPlan fp;
    rc = plan_fused(p, di, &fp);
    if (rc != FRNN_OK) return rc;
    trace("[frnn] %s\n", plan_string(p, path, &fp));
    const size_t rbytes = align256((size_t)slots_of(p.cell) * p.N * p.D * p.D * (p.r_f32 ? 4 : 2));
    char* xw = base + rbytes;
    if (!p.r_f32 && launch_rpack(p, base, st) != hipSuccess) return FRNN_EHIP;
    const void* fn = reinterpret_cast<const void*>(fp.v->fn);
    const size_t wx_elt = p.wx_f32 ? 4 : 2, s0_elt = p.s0_f32 ? 4 : 2;
    // the batch in chunks of at most Bc rows, one launch each (rows never interact)
    for (int b0 = 0; b0 < p.B; b0 += fp.Bc) {
      const int Bch = std::min(fp.Bc, p.B - b0);
      const int groups = p.N * ((Bch + fp.BR - 1) / fp.BR);
      int grid = groups;
      if (!fp.local) grid = ((groups + fp.n_xcd - 1) / fp.n_xcd) * fp.W * fp.n_xcd;
      // exchange words start with tag 0xFFFF, which no step before 65535 polls for (by then
      // every word has been overwritten); the per-die counters after them start at 0xFFFF too
      const size_t xbytes = fp.local ? 0 : (size_t)groups * 2 * fp.BR * p.D * 4;
      if (!fp.local && launch_fill(xw, xbytes + kCtrBytes, st, 0xFFFFu) != hipSuccess) return FRNN_EHIP;
      FusedArgs a;
      std::memset(&a, 0, sizeof(a));
      a.B = Bch; a.T = p.T; a.N = p.N; a.D = p.D;
      a.BR = fp.BR; a.groups = groups; a.W = fp.W; a.n_xcd = fp.n_xcd;
      a.slots = fp.local ? 0 : grid / fp.n_xcd;
      a.ctr = reinterpret_cast<uint32_t*>(xw + xbytes);
      a.xcc_of = 0;
      for (int d = 0; d < kMaxDies; ++d) a.xcc_of |= (uint32_t)(di.xcc_of[d] & 0xF) << (4 * d);
      a.Wx = reinterpret_cast<const char*>(p.Wx) + (long long)b0 * p.wx_sb * (long long)wx_elt;
      a.wx_f32 = p.wx_f32; a.wx_sb = p.wx_sb; a.wx_st = p.wx_st;
      a.R = p.R; a.r_sg = p.r_sg; a.r_sn = p.r_sn; a.r_sd = p.r_sd; a.bias = p.bias;
      a.s0_h = p.s0_h ? reinterpret_cast<const char*>(p.s0_h) + (long long)b0 * p.s0_sb * (long long)s0_elt : nullptr;
      a.s0_c = p.s0_c ? reinterpret_cast<const char*>(p.s0_c) + (long long)b0 * p.s0_sb * (long long)s0_elt : nullptr;
      a.s0_f32 = p.s0_f32; a.s0_sb = p.s0_sb; a.s0_sn = p.s0_sn;
      a.out_h = p.out_h ? p.out_h + (long long)b0 * p.out_sb : nullptr;
      a.out_c = p.out_c ? p.out_c + (long long)b0 * p.out_sb : nullptr;
      a.out_sb = p.out_sb; a.out_st = p.out_st;
      a.last_h = p.last_h ? p.last_h + (long long)b0 * p.last_sb : nullptr;
      a.last_c = p.last_c ? p.last_c + (long long)b0 * p.last_sb : nullptr;
      a.last_sb = p.last_sb; a.last_sn = p.last_sn;
      a.rev_n0 = p.rev_n0;
      a.rpack = base;
      a.xbuf = reinterpret_cast<uint32_t*>(xw);
      a.err = err;
      a.timeout_ticks = (long long)env_int("FRNN_TIMEOUT_MS", 2000) * di.wall_khz;
      a.stall_step = env_int("FRNN_TEST_STALL_STEP", -1);
      void* args[] = {&a};
      if (fp.local) {
        if (hipLaunchKernel(fn, dim3(grid), dim3(fused_threads(fp.ncw)), args, fp.lds, st) != hipSuccess) return FRNN_EHIP;
      } else {
        const int lrc = launch_resident(fn, grid, fused_threads(fp.ncw), fp.lds, args, di.cus, st);
        if (lrc != FRNN_OK) return lrc;
      }
    }
    return FRNN_OK;
  }
  // alternating
  trace("[frnn] %s\n", plan_string(p, path, nullptr));
  const int GS = slots_of(p.cell);
  const size_t elt = p.r_f32 ? 4 : 2;
  AltArgs a;
  std::memset(&a, 0, sizeof(a));
  a.B = p.B; a.T = p.T; a.N = p.N; a.D = p.D; a.cell = p.cell; a.r_is_f32 = p.r_f32;
  a.Wx = p.Wx; a.wx_f32 = p.wx_f32; a.wx_sb = p.wx_sb; a.wx_st = p.wx_st;
  a.R = p.R; a.r_sg = p.r_sg; a.r_sn = p.r_sn; a.r_sd = p.r_sd; a.bias = p.bias;
  a.s0_h = p.s0_h; a.s0_c = p.s0_c; a.s0_f32 = p.s0_f32; a.s0_sb = p.s0_sb; a.s0_sn = p.s0_sn;
  a.out_h = p.out_h; a.out_c = p.out_c; a.out_sb = p.out_sb; a.out_st = p.out_st;
  a.last_h = p.last_h; a.last_c = p.last_c; a.last_sb = p.last_sb; a.last_sn = p.last_sn;
  a.rev_n0 = p.rev_n0;
  char* q = base;
  a.rpack = q; q += align256((size_t)GS * p.N * p.D * p.D * elt);
  a.hbuf[0] = q; q += align256((size_t)p.N * p.B * p.D * elt);
  a.hbuf[1] = q; q += align256((size_t)p.N * p.B * p.D * elt);
  a.ccur = reinterpret_cast<float*>(q);
  const int TPH = GS * p.D / 16;
  if (launch_rpack(p, a.rpack, st) != hipSuccess) return FRNN_EHIP;
  const long long nstate = (long long)p.B * p.N * p.D;
  hipLaunchKernelGGL(alt_init_kernel, dim3((unsigned)std::min<long long>((nstate + 255) / 256, 4096)), dim3(256), 0, st, a);
  const dim3 ggrid(TPH, (p.B + 15) / 16, p.N);
  for (int t = 0; t < p.T; ++t) {
    if (p.r_f32) hipLaunchKernelGGL(alt_step_kernel<true>, ggrid, dim3(256), 0, st, a, t);
    else hipLaunchKernelGGL(alt_step_kernel<false>, ggrid, dim3(256), 0, st, a, t);
  }
  return hipGetLastError() == hipSuccess ? FRNN_OK : FRNN_EHIP;
}

// ----------------------------------------------------------------------------- backward
// Workspace of frnn_bwd after the error word (grows with T: it holds every step's h.R and da).
// K split of the dR GEMM (K = T*B is long and its output small): the parts are summed by the
// scatter kernel. The multi-layer backward's dWi GEMMs take BWD_DR_PARTS parts.
constexpr int BWD_DR_PARTS = 8;

// Rows of the (t, b) operand buffers: T*B padded to whole 32-wide k-tiles of every one of P parts.
size_t bwd_kp(int T, int B, int P = BWD_DR_PARTS) {
  const size_t q = 32 * (size_t)P;
  return ((size_t)T * B + q - 1) / q * q;
}

// K parts of the head-wise dR GEMM (all heads in one launch): eight, doubled (up to 128) while the
// output tiles of all heads times the parts stay under 512 workgroups and a part keeps at least
// 512 of K. Many narrow heads have few output tiles each: twelve heads of 64 units have one 256 x
// 128 tile each, so eight parts would leave the K = T*B sum to 96 workgroups.
int bwd_dr_parts(int T, int B, int N, int D, int G) {
  const long long tiles = (long long)N * ((D + 1 + PJ_BM - 1) / PJ_BM) * ((G * D + PJ_BN - 1) / PJ_BN);
  int P = BWD_DR_PARTS;
  while (P < 128 && tiles * P < 512 && (long long)T * B >= 1024LL * P) P *= 2;
  return P;
}

struct BwdLayout {
  size_t zeros, hprev, hprevT, rt, rpk, hr, da, daT, tmp, dhpart, carry, rec, dstate, xbuf, total;
};

// Fused backward design: groups of BR batch rows of one head on one die, W workgroups each owning
// MT_WG 16-unit tiles of R's rows, (compute waves, K split) over K = G*D.
struct FusedBwdPlan {
  const FusedBwdVariant* v = nullptr;
  int px = 0;                  // 1: the partial-sum design (fused_bwdx_kernel), 0: the da exchange
  int local = 0;               // 1: the single-workgroup fp32 design (fused_bwd_local_kernel)
  fused_bwd_fn fn = nullptr;   // the kernel of the design
  int W = 0, BR = 0, groups = 0, ncw = 0, ks = 0, mtw = 0, ktw = 0, n_xcd = 1, slots = 0, grid = 0, U = 0;
  int ktl = 0;             // k-tiles of R per compute wave kept in LDS (partial-sum design)
  int chunks = 1, Bc = 0;  // the batch runs as `chunks` launches of at most Bc rows
  size_t lds = 0;
};

// The partial-sum design: workgroup w owns units [w*UW, (w+1)*UW) of a head with all their
// gates. Constraints: UW a multiple of 8 (an A fragment stays inside one gate) with G*UW a
// multiple of 32 (whole k-tiles), at most BWDX_MAX_W workgroups (the pollers' words per lane),
// the (row, unit quad) combinations within the compute waves' pollers, the I/O wave's limits and
// an instantiated (waves, tiles, k-tiles) design. Same preference order as the da design.
bool plan_fused_bwdx(int B, int N, int D, int cell, const DevInfo& di, FusedBwdPlan* out) {
  const int G = gates_of(cell);
  const int TPH = D / 16;
  const int slots_per_die = std::max(1, di.cus / di.n_xcd);
  const int force_w = env_int("FRNN_FUSED_BWD_W", 0), force_br = env_int("FRNN_FUSED_BWD_BR", 0);
  const int force_ncw = env_int("FRNN_FUSED_BWD_NCW", 0);
  const int cand[] = {8, 6, 4};
  FusedBwdPlan best;
  bool found = false;
  for (int BR = 1; BR <= FUSED_DIE_MAX_BR; ++BR) {
    if (force_br && BR != force_br) continue;
    for (int W = std::min(BWDX_MAX_W, slots_per_die); W >= 2; --W) {
      if (force_w && W != force_w) continue;
      if (D % W) continue;
      const int UW = D / W;
      if (UW % 8 || (G * UW) % 32) continue;
      const int max_groups = (slots_per_die / W) * di.n_xcd;
      if (max_groups < N) continue;
      const long long bmax = (long long)BR * (max_groups / N);
      const int chunks = (int)((B + bmax - 1) / bmax);
      const int Bc = (B + chunks - 1) / chunks;
      const int groups = N * ((Bc + BR - 1) / BR);
      const int per_die = (groups + di.n_xcd - 1) / di.n_xcd;
      // a step's records fill at most one slot of the I/O wave's LDS ring; its outputs, two
      // 8-byte words per I/O lane
      if (BR * UW * BWD_REC * 4 > BWDX_SLOT || BR * UW > 64 * BWD_EPL_OUT) continue;
      for (const int ncw : cand) {
        if (force_ncw && ncw != force_ncw) continue;
        if (TPH % ncw) continue;
        const int mtw = TPH / ncw, ktw = G * UW / 32;
        if (BR * (UW / 4) > BWDX_CPW * ncw) continue;
        const FusedBwdxVariant* v = find_fused_bwdx(cell, ncw, mtw, ktw);
        if (!v) continue;
        if (found && chunks >= best.chunks) continue;
        const size_t lds = (size_t)fused_bwdx_lds(ktw, BR, UW, ncw, mtw, v->ktl).total;
        if (lds > (size_t)kMaxLds) continue;
        FusedBwdPlan fp;
        fp.px = 1; fp.fn = v->fn; fp.W = W; fp.BR = BR; fp.groups = groups; fp.ncw = ncw; fp.ks = 1; fp.mtw = mtw;
        fp.ktw = ktw; fp.ktl = v->ktl; fp.n_xcd = di.n_xcd; fp.slots = per_die * W; fp.grid = fp.slots * di.n_xcd;
        fp.U = UW; fp.chunks = chunks; fp.Bc = Bc;
        fp.lds = lds;
        best = fp;
        found = true;
        break;
      }
    }
  }
  if (found) *out = best;
  return found;
}

int plan_fused_bwd_da(int B, int N, int D, int cell, const DevInfo& di, FusedBwdPlan* out);

// The single-workgroup design, a head and BR batch rows per workgroup (as many rows
// as the I/O wave's limits allow), the batch in chunks when the groups exceed the CUs.
// bf16 inputs multiply on the bf16 MFMA, fp32 ones on the fp32 MFMA.
int plan_fused_bwd_local(int B, int N, int D, int cell, int f32, const DevInfo& di, FusedBwdPlan* out) {
  const bool bf = !f32;
  const fused_bwd_fn fn = cell == FRNN_CELL_LSTM ? fused_bwd_local_lstm(D, bf)
                          : cell == FRNN_CELL_GRU ? fused_bwd_local_gru(D, bf)
                                                  : fused_bwd_local_elman(D, bf);
  if (!fn || D / 16 > BWDL_NCW) return FRNN_EUNSUPPORTED;
  const int G = gates_of(cell);
  FusedBwdPlan fp;
  fp.local = 1; fp.fn = fn; fp.W = 1; fp.ncw = BWDL_NCW; fp.ks = 1; fp.mtw = 1; fp.ktw = G * D / (bf ? 32 : 4);
  fp.BR = std::max(1, std::min(B, fused_bwdl_max_br(D)));
  const long long bmax = (long long)fp.BR * std::max(1, di.cus / N);
  if (di.cus < N) return FRNN_EUNSUPPORTED;
  fp.chunks = (int)((B + bmax - 1) / bmax);
  fp.Bc = (B + fp.chunks - 1) / fp.chunks;
  fp.groups = N * ((fp.Bc + fp.BR - 1) / fp.BR);
  fp.grid = fp.groups;
  fp.n_xcd = 1; fp.U = D;
  fp.lds = (size_t)fused_bwdl_lds(G, D, fp.BR, bf).total;
  *out = fp;
  return FRNN_OK;
}

// Heads of at most 64 units take the single-workgroup design: on the bf16 MFMA it measured 1.2-2.6x
// faster than the partial-sum design for every cell (B x N from 16 x 1 to 256 x 4, T = 512), and
// fp32 operands have no other. Wider bf16 heads take the partial-sum design where it has a plan
// with no more launches than the da design, else the da design. FRNN_FUSED_BWD_PX pins a design:
// 1 the partial sums, 0 the da exchange, 2 the single workgroup.
int plan_fused_bwd(int B, int N, int D, int cell, int f32, const DevInfo& di, FusedBwdPlan* out) {
  if (f32) return plan_fused_bwd_local(B, N, D, cell, f32, di, out);
  const int design = env_int("FRNN_FUSED_BWD_PX", -1);
  if (design == 2) return plan_fused_bwd_local(B, N, D, cell, f32, di, out);
  if (design < 0 && plan_fused_bwd_local(B, N, D, cell, f32, di, out) == FRNN_OK) return FRNN_OK;
  if (!di.periodic || D % 32 != 0) return design < 0 ? plan_fused_bwd_local(B, N, D, cell, f32, di, out) : FRNN_EUNSUPPORTED;
  FusedBwdPlan px, da;
  const bool has_px = design != 0 && plan_fused_bwdx(B, N, D, cell, di, &px);
  const bool has_da = design != 1 && plan_fused_bwd_da(B, N, D, cell, di, &da) == FRNN_OK;
  if (has_px && (!has_da || px.chunks <= da.chunks)) {
    *out = px;
    return FRNN_OK;
  }
  if (has_da) {
    *out = da;
    return FRNN_OK;
  }
  return design < 0 ? plan_fused_bwd_local(B, N, D, cell, f32, di, out) : FRNN_EUNSUPPORTED;
}

int plan_fused_bwd_da(int B, int N, int D, int cell, const DevInfo& di, FusedBwdPlan* out) {
  const int G = gates_of(cell);
  const int TPH = D / 16, KT = G * D / 32;
  const int slots_per_die = std::max(1, di.cus / di.n_xcd);
  const int force_w = env_int("FRNN_FUSED_BWD_W", 0), force_br = env_int("FRNN_FUSED_BWD_BR", 0);
  const int force_ncw = env_int("FRNN_FUSED_BWD_NCW", 0);
  const int cand[][2] = {{8, 8}, {6, 6}, {4, 4}, {4, 2}};
  // Fewest launches first (a batch whose groups cannot all be co-resident runs in chunks of rows,
  // one launch each), then fewest batch rows per group, then the widest split, then the
  // (compute waves, K split) order above.
  FusedBwdPlan best;
  bool found = false;
  for (int BR = 1; BR <= FUSED_DIE_MAX_BR; ++BR) {
    if (force_br && BR != force_br) continue;
    for (int W = std::min(32, slots_per_die); W >= 2; --W) {
      if (force_w && W != force_w) continue;
      const int max_groups = (slots_per_die / W) * di.n_xcd;
      if (TPH % W || max_groups < N) continue;
      const long long bmax = (long long)BR * (max_groups / N);
      const int chunks = (int)((B + bmax - 1) / bmax);
      const int Bc = (B + chunks - 1) / chunks;
      const int groups = N * ((Bc + BR - 1) / BR);
      const int per_die = (groups + di.n_xcd - 1) / di.n_xcd;
      const int mt_wg = TPH / W, U = mt_wg * 16;
      // the I/O wave moves at most 64 * BWD_EPL_IN record words and 64 * BWD_EPL_OUT output words
      if (BR * U * BWD_REC / 2 > 64 * BWD_EPL_IN || BR * U > 64 * BWD_EPL_OUT) continue;
      for (const auto& nk : cand) {
        const int ncw = nk[0], ks = nk[1];
        if (force_ncw && ncw != force_ncw) continue;
        const int ms = ncw / ks;
        if (mt_wg % ms || KT % ks) continue;
        const int mtw = mt_wg / ms, ktw = KT / ks;
        const FusedBwdVariant* v = find_fused_bwd(cell, ncw, ks, mtw, ktw);
        if (!v || BR > fused_max_br(ks, mtw)) continue;
        if (found && chunks >= best.chunks) continue;  // earlier candidates win ties
        FusedBwdPlan fp;
        fp.v = v; fp.fn = v->fn; fp.W = W; fp.BR = BR; fp.groups = groups; fp.ncw = ncw; fp.ks = ks; fp.mtw = mtw;
        fp.ktw = ktw; fp.n_xcd = di.n_xcd; fp.slots = per_die * W; fp.grid = fp.slots * di.n_xcd; fp.U = U;
        fp.chunks = chunks; fp.Bc = Bc;
        fp.lds = (size_t)fused_bwd_lds(ncw, ks, mtw, ktw, BR, U).total;
        best = fp;
        found = true;
        break;
      }
    }
  }
  if (!found) return FRNN_EUNSUPPORTED;
  *out = best;
  return FRNN_OK;
}

BwdLayout bwd_layout(int B, int T, int N, int D, int cell, int f32, int path) {
  const size_t G = gates_of(cell), elt = f32 ? 4 : 2;
  const int P = bwd_dr_parts(T, B, N, D, (int)G);
  const size_t Kp = bwd_kp(T, B, P);
  BwdLayout L;
  size_t q = 0;
  L.zeros = q;  q += 256;
  L.hprev = q;  q += align256((size_t)N * Kp * D * elt);
  L.hprevT = q; q += align256((size_t)N * (D + 1) * Kp * elt);
  L.rt = q;     q += align256((size_t)N * G * D * D * elt);
  L.rpk = q;    q += align256((size_t)N * G * D * D * elt);
  L.hr = q;     q += align256((size_t)N * T * B * G * D * 4);
  L.da = q;     q += align256((size_t)N * Kp * G * D * elt);
  L.daT = q;    q += align256((size_t)N * G * D * Kp * elt);
  L.tmp = q;    q += align256((size_t)P * N * (D + 1) * G * D * 4);
  L.dhpart = q; q += align256((size_t)BWD_KS * B * N * D * 4);
  L.carry = q;  q += align256((size_t)B * N * D * 4);
  L.rec = L.dstate = L.xbuf = q;
  if (path == FRNN_PATH_FUSED) {
    L.rec = q;    q += align256((size_t)T * B * N * D * BWD_REC * 4);
    L.dstate = q; q += align256((size_t)T * B * N * D * 2 * 4);
    // exchange words: groups * BR <= N * (B + 3) rows (BR <= 4), two parities, G*D words a row
    // (da design) or W*D words a row (partial-sum design, W <= BWDX_MAX_W)
    L.xbuf = q;
    q += align256((size_t)2 * N * (B + FUSED_DIE_MAX_BR - 1) * std::max<size_t>(G, BWDX_MAX_W) * D * 4) + kCtrBytes;
  }
  L.total = q;
  return L;
}

// The alternating backward's step in one launch (bwd_step_kernel: each workgroup contracts a whole
// K = G*D) where K is short, else two (bwd_gate_kernel, then bwd_dh_kernel split over K); the
// crossover measured between G*D = 1024 and 2048. FRNN_ALT_BWD_ONE_LAUNCH=0/1 pins either.
bool bwd_one_launch(int G, int D) {
  const int pin = env_int("FRNN_ALT_BWD_ONE_LAUNCH", -1);
  return pin >= 0 ? pin != 0 : G * D <= 1024;
}

std::string bwd_plan_string(const frnn_desc* d, int path, const FusedBwdPlan* fp = nullptr) {
  char buf[512];
  if (path == FRNN_PATH_FUSED && fp) {
    std::snprintf(buf, sizeof(buf),
                  "backward path=fused design=%s cell=%s dtype=%s B=%d T=%d N=%d D=%d BR=%d groups=%d W=%d "
                  "NCW=%d KS=%d MTW=%d KTW=%d%s dies=%d slots/die=%d grid=%d lds=%zu chunks=%d rows/chunk=%d",
                  fp->local ? "workgroup-local" : fp->px ? "die-local-partials" : "die-local", cell_name(d->cell),
                  d->in_dtype == FRNN_F32 ? "f32" : "bf16", d->B, d->T, d->N, d->D, fp->BR, fp->groups, fp->W, fp->ncw, fp->ks, fp->mtw,
                  fp->ktw, fp->ktl > 0 ? (" KTL=" + std::to_string(fp->ktl)).c_str() : "", fp->n_xcd, fp->slots, fp->grid,
                  fp->lds, fp->chunks, fp->Bc);
    return std::string(buf);
  }
  const int G = gates_of(d->cell);
  const long long Kp = (long long)bwd_kp(d->T, d->B, bwd_dr_parts(d->T, d->B, d->N, d->D, G));
  std::snprintf(buf, sizeof(buf),
                "backward path=%s cell=%s dtype=%s B=%d T=%d N=%d D=%d hr_gemm=%lldx%dx%d dR_gemm=%dx%dx%lld "
                "step_launches=%d",
                path == FRNN_PATH_FUSED ? "fused" : "alternating", cell_name(d->cell),
                d->in_dtype == FRNN_F32 ? "f32" : "bf16", d->B, d->T, d->N, d->D, (long long)d->T * d->B, G * d->D,
                d->D, d->D + 1, G * d->D, Kp, path == FRNN_PATH_FUSED ? 1 : bwd_one_launch(G, d->D) ? d->T : 2 * d->T);
  return std::string(buf);
}

// Launch bwd_gate_kernel or bwd_step_kernel (step t) or bwd_record_kernel (rec) instantiated for
// the cell, the operand dtype and the Wx dtype.
enum BwdCellKernel { kBwdGate, kBwdStep, kBwdRecord };

template <int CELL, bool F32, bool WXF32>
void launch_bwd_cell_kernel_t(BwdCellKernel k, dim3 grid, dim3 block, hipStream_t st, const BwdArgs& a, int t, float* rec) {
  if (k == kBwdGate) hipLaunchKernelGGL((bwd_gate_kernel<CELL, F32, WXF32>), grid, block, 0, st, a, t);
  else if (k == kBwdStep) hipLaunchKernelGGL((bwd_step_kernel<CELL, F32, WXF32>), grid, block, 0, st, a, t);
  else hipLaunchKernelGGL((bwd_record_kernel<CELL, F32, WXF32>), grid, block, 0, st, a, rec);
}

template <int CELL>
void launch_bwd_cell_kernel_c(BwdCellKernel k, bool f32, bool wx_f32, dim3 grid, dim3 block, hipStream_t st,
                              const BwdArgs& a, int t, float* rec) {
  if (f32) launch_bwd_cell_kernel_t<CELL, true, true>(k, grid, block, st, a, t, rec);  // fp32 inputs: Wx fp32 too
  else if (wx_f32) launch_bwd_cell_kernel_t<CELL, false, true>(k, grid, block, st, a, t, rec);
  else launch_bwd_cell_kernel_t<CELL, false, false>(k, grid, block, st, a, t, rec);
}

void launch_bwd_cell_kernel(BwdCellKernel k, int cell, bool f32, bool wx_f32, dim3 grid, dim3 block, hipStream_t st,
                            const BwdArgs& a, int t, float* rec) {
  if (cell == FRNN_CELL_LSTM) launch_bwd_cell_kernel_c<CELL_LSTM>(k, f32, wx_f32, grid, block, st, a, t, rec);
  else if (cell == FRNN_CELL_GRU) launch_bwd_cell_kernel_c<CELL_GRU>(k, f32, wx_f32, grid, block, st, a, t, rec);
  else launch_bwd_cell_kernel_c<CELL_ELMAN>(k, f32, wx_f32, grid, block, st, a, t, rec);
}

// The single-workgroup design on an Elman cell needs no records: its I/O wave loads h and ds_h
// itself (16-byte rows, which the boundary's alignment rules guarantee; checked again here), and
// then no step needs h.R either. FRNN_BWD_ELMAN_RAW=0 pins compact records.
bool bwd_elman_raw(const BwdArgs& a, const FusedBwdPlan& fp) {
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  return fp.local && a.cell == FRNN_CELL_ELMAN && al16(a.st_h) && (!a.ds_h || al16(a.ds_h)) &&
         (!a.dl_h || al16(a.dl_h)) && a.st_sb % 4 == 0 && a.st_st % 4 == 0 && a.last_sb % 4 == 0 && a.D % 4 == 0 &&
         env_int("FRNN_BWD_ELMAN_RAW", 1) != 0;
}

// The fused serial part: records of every step, the persistent kernel, then dWx / da / carries.
int run_fused_bwd(int cell, const BwdArgs& a, const FusedBwdPlan& fp, const DevInfo& di, char* base,
                  const BwdLayout& L, hipStream_t st) {
  const long long total = (long long)a.T * a.B * a.N * a.D;
  const unsigned pgrid = (unsigned)((total + 255) / 256);
  float* rec = reinterpret_cast<float*>(base + L.rec);
  float* dstate = reinterpret_cast<float*>(base + L.dstate);
  const bool f32 = a.f32 != 0;
  // the single-workgroup design keeps an Elman cell's records compact (two coefficients)
  const bool compact = fp.local && cell == FRNN_CELL_ELMAN;
  const int rec_f = compact ? 2 : BWD_REC;
  // ... or none at all (bwd_elman_raw)
  const bool raw = compact && bwd_elman_raw(a, fp);
  if (raw) {
    // no records
  } else if (compact) {
    if (f32) hipLaunchKernelGGL((bwd_record_kernel<CELL_ELMAN, true, true, 2>), dim3(pgrid), dim3(256), 0, st, a, rec);
    else if (a.wx_f32) hipLaunchKernelGGL((bwd_record_kernel<CELL_ELMAN, false, true, 2>), dim3(pgrid), dim3(256), 0, st, a, rec);
    else hipLaunchKernelGGL((bwd_record_kernel<CELL_ELMAN, false, false, 2>), dim3(pgrid), dim3(256), 0, st, a, rec);
  } else {
    launch_bwd_cell_kernel(kBwdRecord, cell, f32, a.wx_f32, dim3(pgrid), dim3(256), st, a, 0, rec);
  }
  const void* fn = reinterpret_cast<const void*>(fp.fn);
  // the single-workgroup design takes R's fragments in its inputs' type: the packed operand
  const void* rpk_local = a.rpk;
  // the batch in chunks of at most Bc rows, one launch each (rows never interact)
  for (int b0 = 0; b0 < a.B; b0 += fp.Bc) {
    const int Bch = std::min(fp.Bc, a.B - b0);
    const int groups = a.N * ((Bch + fp.BR - 1) / fp.BR);
    if (fp.local) {  // single-workgroup design: a workgroup per group, no exchange, no placement
      FusedBwdArgs f;
      std::memset(&f, 0, sizeof(f));
      f.B = Bch; f.Bs = a.B; f.T = a.T; f.N = a.N; f.D = a.D;
      f.BR = fp.BR; f.groups = groups; f.W = 1; f.n_xcd = 1;
      f.rpk = rpk_local;
      f.rec = rec + (size_t)b0 * a.N * a.D * rec_f;
      f.dstate = dstate + (size_t)b0 * a.N * a.D * 2;
      f.bbase = b0;
      f.dWx = a.dWx; f.wx_sb = a.wx_sb; f.wx_st = a.wx_st;
      f.da = a.da; f.Kp = a.Kp; f.f32op = a.f32; f.carry = a.carry;
      f.raw = raw ? 1 : 0;
      f.st_h = a.st_h; f.ds_h = a.ds_h; f.dl_h = a.dl_h; f.zeros = a.zeros;
      f.st_sb = a.st_sb; f.st_st = a.st_st; f.last_sb = a.last_sb;
      f.err = reinterpret_cast<int*>(base - kErrBytes);
      f.stall_step = -1;
      void* args[] = {&f};
      if (hipLaunchKernel(fn, dim3(groups), dim3((BWDL_NCW + 1) * 64), args, fp.lds, st) != hipSuccess) return FRNN_EHIP;
      continue;
    }
    const int grid = ((groups + fp.n_xcd - 1) / fp.n_xcd) * fp.W * fp.n_xcd;
    const size_t xbytes = (size_t)groups * 2 * fp.BR * (fp.px ? fp.W : gates_of(cell)) * a.D * 4;
    if (launch_fill(base + L.xbuf, xbytes + kCtrBytes, st, 0xFFFFu) != hipSuccess) return FRNN_EHIP;
    FusedBwdArgs f;
    std::memset(&f, 0, sizeof(f));
    f.B = Bch; f.Bs = a.B; f.T = a.T; f.N = a.N; f.D = a.D;
    f.BR = fp.BR; f.groups = groups; f.W = fp.W; f.n_xcd = fp.n_xcd; f.slots = grid / fp.n_xcd;
    f.ctr = reinterpret_cast<uint32_t*>(base + L.xbuf + xbytes);
    f.xcc_of = 0;
    for (int k = 0; k < kMaxDies; ++k) f.xcc_of |= (uint32_t)(di.xcc_of[k] & 0xF) << (4 * k);
    f.rpk = a.rpk;
    f.rec = rec + (size_t)b0 * a.N * a.D * BWD_REC;
    f.dstate = dstate + (size_t)b0 * a.N * a.D * 2;
    f.bbase = b0;
    f.dWx = a.dWx; f.wx_sb = a.wx_sb; f.wx_st = a.wx_st;
    f.da = a.da; f.Kp = a.Kp; f.f32op = a.f32; f.carry = a.carry;
    f.xbuf = reinterpret_cast<uint32_t*>(base + L.xbuf);
    f.err = reinterpret_cast<int*>(base - kErrBytes);
    f.timeout_ticks = (long long)env_int("FRNN_TIMEOUT_MS", 2000) * di.wall_khz;
    f.stall_step = env_int("FRNN_TEST_STALL_STEP", -1);
    void* args[] = {&f};
    const int lrc = launch_resident(fn, grid, fused_threads(fp.ncw), fp.lds, args, di.cus, st);
    if (lrc != FRNN_OK) return lrc;
  }
  if (fp.local || fp.px) {
    // the serial kernel stored dWx, da and the carries of time step 0 (an Elman cell's are zero
    // from the start)
  } else if (f32) {
    if (cell == FRNN_CELL_LSTM) hipLaunchKernelGGL((bwd_post_kernel<CELL_LSTM, true>), dim3(pgrid), dim3(256), 0, st, a, rec, dstate);
    else if (cell == FRNN_CELL_GRU) hipLaunchKernelGGL((bwd_post_kernel<CELL_GRU, true>), dim3(pgrid), dim3(256), 0, st, a, rec, dstate);
    else hipLaunchKernelGGL((bwd_post_kernel<CELL_ELMAN, true>), dim3(pgrid), dim3(256), 0, st, a, rec, dstate);
  } else {
    if (cell == FRNN_CELL_LSTM) hipLaunchKernelGGL((bwd_post_kernel<CELL_LSTM, false>), dim3(pgrid), dim3(256), 0, st, a, rec, dstate);
    else if (cell == FRNN_CELL_GRU) hipLaunchKernelGGL((bwd_post_kernel<CELL_GRU, false>), dim3(pgrid), dim3(256), 0, st, a, rec, dstate);
    else hipLaunchKernelGGL((bwd_post_kernel<CELL_ELMAN, false>), dim3(pgrid), dim3(256), 0, st, a, rec, dstate);
  }
  return hipGetLastError() == hipSuccess ? FRNN_OK : FRNN_EHIP;
}

// A backward problem with explicit element strides: G gates of N heads of D units; the gates of
// Wx and dWx lie N*D elements apart; dstates shares the states' strides.
struct BwdProblem {
  int B, T, N, D, cell;
  int f32;     // R, bias, initial states and the MFMA operands fp32 (else bf16)
  int wx_f32;  // Wx fp32 (else as f32)
  const void* Wx;
  long long wx_sb, wx_st;
  const void* R;
  long long r_sg, r_sn, r_sd;
  const void* bias;
  const void* s0_h;
  const void* s0_c;
  long long s0_sb;
  const float* st_h;
  const float* st_c;
  long long st_sb, st_st;
  const float* ds_h;
  const float* ds_c;
  const float* dl_h;
  const float* dl_c;
  long long last_sb;
  float* dWx;
  float* dR;
  long long dr_sg, dr_sn, dr_sd;
  float* db;     // [G][N][D]
  float* ds0_h;  // [B][N][D]
  float* ds0_c;
};

// The backward of a validated problem with T > 0 on `path` (the fused plan given for the fused
// path). `base` is the workspace after its error word, laid out as L.
int run_backward(const BwdProblem& q, int path, const FusedBwdPlan& fbp, const DevInfo& di, char* base,
                 const BwdLayout& L, hipStream_t st) {
  const int B = q.B, T = q.T, N = q.N, D = q.D, G = gates_of(q.cell), f32 = q.f32;
  const long long BND = (long long)B * N * D;
  const size_t elt = f32 ? 4 : 2;
  const unsigned sgrid = (unsigned)((BND + 255) / 256);
  int rc = FRNN_OK;
  const int parts = bwd_dr_parts(T, B, N, D, G);
  const int Kp = (int)bwd_kp(T, B, parts);
  BwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.B = B; a.T = T; a.N = N; a.D = D; a.cell = q.cell; a.f32 = f32; a.wx_f32 = f32 || q.wx_f32; a.Kp = Kp;
  a.Wx = q.Wx; a.wx_sb = q.wx_sb; a.wx_st = q.wx_st;
  a.R = q.R; a.r_sg = q.r_sg; a.r_sn = q.r_sn; a.r_sd = q.r_sd;
  a.bias = q.bias;
  a.s0_h = q.s0_h; a.s0_c = q.s0_c; a.s0_sb = q.s0_sb;
  a.st_h = q.st_h; a.st_c = q.st_c; a.st_sb = q.st_sb; a.st_st = q.st_st;
  a.ds_h = q.ds_h; a.ds_c = q.ds_c;
  a.dl_h = q.dl_h; a.dl_c = q.dl_c; a.last_sb = q.last_sb;
  a.dWx = q.dWx;
  a.ds0_h = q.ds0_h; a.ds0_c = q.ds0_c;
  a.hprev = base + L.hprev;
  a.hr = reinterpret_cast<const float*>(base + L.hr);
  a.da = base + L.da;
  a.zeros = reinterpret_cast<const float*>(base + L.zeros);
  a.rpk = base + L.rpk;
  a.dhpart = reinterpret_cast<float*>(base + L.dhpart);
  a.ks = std::min(BWD_KS, G * D / (f32 ? 4 : 32));
  a.carry = reinterpret_cast<float*>(base + L.carry);
  char* hT = base + L.hprevT;
  char* rt = base + L.rt;
  char* daT = base + L.daT;
  float* tmp = reinterpret_cast<float*>(base + L.tmp);
  float* hr = reinterpret_cast<float*>(base + L.hr);
  // carried gradients start at zero
  if (launch_fill(base + L.zeros, 256, st) != hipSuccess ||
      launch_fill(a.dhpart, (size_t)BWD_KS * BND * 4, st) != hipSuccess || launch_fill(a.carry, (size_t)BND * 4, st) != hipSuccess)
    return FRNN_EHIP;
  // da's rows past T*B (padding to whole k-tiles of every dR part) must read zero
  if ((size_t)Kp > (size_t)T * B) {
    for (int n = 0; n < N; ++n)
      if (launch_fill(static_cast<char*>(a.da) + ((size_t)n * Kp + (size_t)T * B) * G * D * elt,
                      ((size_t)Kp - (size_t)T * B) * G * D * elt, st) != hipSuccess)
        return FRNN_EHIP;
  }
  // 1. h_{t-1} for every step, R^T, and h.R for every step (none of it where the serial part reads
  // no records: the dR GEMM's h^T then comes straight from the states)
  const bool no_hr = path == FRNN_PATH_FUSED && bwd_elman_raw(a, fbp);
  const bool hT_direct = no_hr && !f32;
  if (!hT_direct)
    hipLaunchKernelGGL(bwd_hprev_kernel, dim3((unsigned)std::min<long long>(((long long)N * Kp * (D / 8) + 255) / 256, 65536)),
                       dim3(256), 0, st, a);
  // R_g^T of every (head, gate): one launch per gate over the heads, or per head over the gates,
  // whichever makes fewer launches
  const bool by_head = N >= G;
  for (int i = 0; i < (no_hr ? 0 : by_head ? G : N); ++i) {
    const int g = by_head ? i : 0, n = by_head ? 0 : i;
    const size_t src = (size_t)g * a.r_sg + (size_t)n * a.r_sn, dst = ((size_t)n * G + g) * D * D;
    const long long src_z = by_head ? a.r_sn : a.r_sg, dst_z = by_head ? (long long)G * D * D : (long long)D * D;
    if (f32)
      launch_transpose<uint32_t>(reinterpret_cast<const uint32_t*>(q.R) + src, a.r_sd, D, D,
                                 reinterpret_cast<uint32_t*>(rt) + dst, D, st, by_head ? N : G, src_z, dst_z);
    else
      launch_transpose<uint16_t>(reinterpret_cast<const uint16_t*>(q.R) + src, a.r_sd, D, D,
                                 reinterpret_cast<uint16_t*>(rt) + dst, D, st, by_head ? N : G, src_z, dst_z);
  }
  // h.R of every head in one launch
  if (!no_hr && launch_gemm(f32, T * B, G * D, D, base + L.hprev, D, rt, D, hr, (long long)G * D, st, 1, 0, 0, 0, false, N,
                            (long long)Kp * D, (long long)G * D * D, (long long)T * B * G * D) != hipSuccess)
    return FRNN_EHIP;
  // 2. the serial part (R packed once as the dh kernels' A fragments)
  {
    const long long np = (long long)N * (D / 16) * (G * D / (f32 ? 4 : 32)) * 64;
    hipLaunchKernelGGL(bwd_rpack_kernel, dim3((unsigned)std::min<long long>((np + 255) / 256, 65536)), dim3(256), 0, st, a,
                       (void*)(base + L.rpk));
  }
  const dim3 hgrid(D / 16, a.ks, ((B + 15) / 16) * N);
  if (path == FRNN_PATH_FUSED) {
    rc = run_fused_bwd(q.cell, a, fbp, di, base, L, st);
    if (rc != FRNN_OK) return rc;
  } else if (bwd_one_launch(G, D)) {
    // one launch per step: the contraction of step t+1's da with R^T, the step's gradients as its
    // epilogue
    const dim3 tgrid(D / 16, 1, ((B + 15) / 16) * N);
    for (int t = T - 1; t >= 0; --t)
      launch_bwd_cell_kernel(kBwdStep, q.cell, f32, a.wx_f32, tgrid, dim3(BWD_STEP_WAVES * 64), st, a, t, nullptr);
  } else {
    // per step: the step's gradients, then their contraction with R^T (in K-split parts) for the
    // step before
    const dim3 g64((unsigned)((BND + 63) / 64)), b64(64);
    for (int t = T - 1; t >= 0; --t) {
      launch_bwd_cell_kernel(kBwdGate, q.cell, f32, a.wx_f32, g64, b64, st, a, t, nullptr);
      if (t == 0) break;  // step 0's contraction is the one below
      if (f32) hipLaunchKernelGGL(bwd_dh_kernel<true>, hgrid, dim3(256), 0, st, a, t);
      else hipLaunchKernelGGL(bwd_dh_kernel<false>, hgrid, dim3(256), 0, st, a, t);
    }
  }
  // the gradient that reaches the initial state through R: one more contraction, of step 0's da
  if (f32) hipLaunchKernelGGL(bwd_dh_kernel<true>, hgrid, dim3(256), 0, st, a, 0);
  else hipLaunchKernelGGL(bwd_dh_kernel<false>, hgrid, dim3(256), 0, st, a, 0);
  hipLaunchKernelGGL(bwd_final_kernel, dim3(sgrid), dim3(256), 0, st, a);
  if (hipGetLastError() != hipSuccess) return FRNN_EHIP;
  // 3. dR and db: per head, [D+1 rows: h^T and ones] x [G*D columns of da], over K = T*B
  if (q.dR || q.db) {
    // h^T and da^T of every head, one launch each
    const long long h_z = (long long)Kp * D, ht_z = (long long)(D + 1) * Kp;
    const long long d_z = (long long)Kp * G * D, dt_z = (long long)G * D * Kp;
    if (hT_direct) {
      hipLaunchKernelGGL(bwd_hprevT_kernel, dim3((D + 63) / 64, std::min(Kp / 64, 65535), N), dim3(256), 0, st, a,
                         reinterpret_cast<uint16_t*>(hT));
      launch_transpose<uint16_t>(reinterpret_cast<const uint16_t*>(a.da), (long long)G * D, Kp, G * D,
                                 reinterpret_cast<uint16_t*>(daT), Kp, st, N, d_z, dt_z);
    } else if (f32) {
      launch_transpose<uint32_t>(reinterpret_cast<const uint32_t*>(a.hprev), D, Kp, D, reinterpret_cast<uint32_t*>(hT), Kp,
                                 st, N, h_z, ht_z);
      launch_transpose<uint32_t>(reinterpret_cast<const uint32_t*>(a.da), (long long)G * D, Kp, G * D,
                                 reinterpret_cast<uint32_t*>(daT), Kp, st, N, d_z, dt_z);
    } else {
      launch_transpose<uint16_t>(reinterpret_cast<const uint16_t*>(a.hprev), D, Kp, D, reinterpret_cast<uint16_t*>(hT), Kp,
                                 st, N, h_z, ht_z);
      launch_transpose<uint16_t>(reinterpret_cast<const uint16_t*>(a.da), (long long)G * D, Kp, G * D,
                                 reinterpret_cast<uint16_t*>(daT), Kp, st, N, d_z, dt_z);
    }
    hipLaunchKernelGGL(bwd_ones_row_kernel, dim3((unsigned)std::min<long long>(((long long)N * Kp + 255) / 256, 4096)),
                       dim3(256), 0, st, hT, N, D, Kp, f32);
    // K split into equal parts (bwd_dr_parts), all parts of all heads in one launch, summed in
    // order by the scatter kernel
    const int kpart = Kp / parts;
    const long long ptot = (long long)N * (D + 1) * G * D;
    if (launch_gemm(f32, D + 1, G * D, kpart, hT, Kp, daT, Kp, tmp, (long long)G * D, st, parts, kpart, kpart, ptot, false,
                    N, ht_z, dt_z, (long long)(D + 1) * G * D) != hipSuccess)
      return FRNN_EHIP;
    const long long nt = ptot / 4;
    hipLaunchKernelGGL(bwd_scatter_kernel, dim3((unsigned)std::min<long long>((nt + 255) / 256, 65536)), dim3(256), 0, st,
                       tmp, parts, N, D, G, q.dR, q.dr_sg, q.dr_sn, q.dr_sd, q.db);
  }
  return hipGetLastError() == hipSuccess ? FRNN_OK : FRNN_EHIP;
}


bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u); }

// Element strides of a description, its dense defaults filled in where it gives 0.
struct Strides {
  long long wx_sb, wx_st, st_ss, st_sb, st_st, r_sg, r_sn, r_sd;
};

Strides strides_of(const frnn_desc* d) {
  const long long T = d->T, N = d->N, D = d->D, B = d->B, G = gates_of(d->cell);
  Strides s;
  s.wx_sb = d->wx_sb ? d->wx_sb : T * G * N * D;
  s.wx_st = d->wx_st ? d->wx_st : G * N * D;
  s.st_ss = d->st_ss ? d->st_ss : B * T * N * D;
  s.st_sb = d->st_sb ? d->st_sb : T * N * D;
  s.st_st = d->st_st ? d->st_st : N * D;
  s.r_sg = d->r_sg ? d->r_sg : N * D * D;
  s.r_sn = d->r_sn ? d->r_sn : D * D;
  s.r_sd = d->r_sd ? d->r_sd : D;
  return s;
}

int validate_desc(const frnn_desc* d, int path) {
  if (!d) return FRNN_EINVAL;
  if (d->reserved != 0) return FRNN_EINVAL;
  if (d->B < 1 || d->N < 1 || d->D < 1 || d->T < 0) return FRNN_EINVAL;
  if (d->cell != FRNN_CELL_LSTM && d->cell != FRNN_CELL_ELMAN && d->cell != FRNN_CELL_GRU) return FRNN_EINVAL;
  if (d->in_dtype != FRNN_F32 && d->in_dtype != FRNN_BF16) return FRNN_EINVAL;
  if (d->out_dtype != FRNN_F32 && d->out_dtype != FRNN_BF16) return FRNN_EINVAL;
  if (path != FRNN_PATH_ALTERNATING && path != FRNN_PATH_FUSED) return FRNN_EINVAL;
  const long long elems = (long long)d->B * d->T * gates_of(d->cell) * d->N * d->D;
  if (elems < 0 || elems > (1LL << 40)) return FRNN_EINVAL;
  // strides: Wx and states rows and steps keep 8-byte (bf16) / 16-byte (fp32) alignment of the
  // kernels' vector accesses; R's are offsets and must not be negative; every offset fits in 2^40
  for (long long v : {d->wx_sb, d->wx_st, d->st_ss, d->st_sb, d->st_st}) {
    if (v % 4 != 0) return FRNN_EINVAL;
    if (v > (1LL << 40) || v < -(1LL << 40)) return FRNN_EINVAL;
  }
  for (long long v : {d->r_sg, d->r_sn, d->r_sd})
    if (v < 0 || v > (1LL << 40)) return FRNN_EINVAL;
  if (d->out_dtype != FRNN_F32) return FRNN_EUNSUPPORTED;
  if (d->D % 32 != 0 || d->D > 1024) return FRNN_EUNSUPPORTED;
  return FRNN_OK;
}

Problem problem_from_desc(const frnn_desc* d, const void* Wx, const void* R, const void* b, const void* s0,
                          void* states, void* last) {
  Problem p;
  std::memset(&p, 0, sizeof(p));
  const long long B = d->B, N = d->N, D = d->D;
  const int f32 = d->in_dtype == FRNN_F32;
  const size_t elt = f32 ? 4 : 2;
  const Strides s = strides_of(d);
  p.B = d->B; p.T = d->T; p.N = d->N; p.D = d->D; p.cell = d->cell; p.r_f32 = f32;
  p.Wx = Wx; p.wx_f32 = f32; p.wx_sb = s.wx_sb; p.wx_st = s.wx_st;
  p.R = R; p.r_sg = s.r_sg; p.r_sn = s.r_sn; p.r_sd = s.r_sd;
  p.bias = b;
  p.s0_h = s0;
  p.s0_c = (s0 && d->cell == FRNN_CELL_LSTM) ? reinterpret_cast<const char*>(s0) + (size_t)B * N * D * elt : nullptr;
  p.s0_f32 = f32; p.s0_sb = N * D; p.s0_sn = D;
  float* st = reinterpret_cast<float*>(states);
  p.out_h = st;
  p.out_c = (st && d->cell == FRNN_CELL_LSTM) ? st + s.st_ss : nullptr;
  p.out_sb = s.st_sb; p.out_st = s.st_st;
  float* ls = reinterpret_cast<float*>(last);
  p.last_h = ls;
  p.last_c = (ls && d->cell == FRNN_CELL_LSTM) ? ls + B * N * D : nullptr;
  p.last_sb = N * D; p.last_sn = D;
  p.rev_n0 = d->N;
  return p;
}

}  // namespace

// ============================================================================= C ABI
extern "C" {

int frnn_abi_version(void) { return FRNN_ABI_VERSION; }

int frnn_init(void) { return init_device(); }

const char* frnn_status_str(int s) {
  switch (s) {
    case FRNN_OK: return "ok";
    case FRNN_EINVAL: return "invalid argument";
    case FRNN_EUNSUPPORTED: return "unsupported by this build (dtype, head dimension or path)";
    case FRNN_EWORKSPACE: return "workspace missing or too small";
    case FRNN_ENORESIDENT: return "persistent grid cannot be co-resident on this device";
    case FRNN_EHIP: return "HIP runtime error";
    case FRNN_ETIMEOUT: return "a bounded inter-workgroup wait ran out on the device";
    case FRNN_EPLACEMENT: return "a workgroup ran on a different accelerator die than planned";
    case FRNN_ENODEVICE: return "no usable gfx950 device";
    case FRNN_ENOINIT: return "frnn_init() has not prepared the current device";
    default: return "unknown status";
  }
}

int frnn_workspace_bytes(const frnn_desc* d, int path, size_t* bytes) {
  const int rc = validate_desc(d, path);
  if (rc != FRNN_OK) return rc;
  if (!bytes) return FRNN_EINVAL;
  *bytes = kErrBytes + rec_scratch_bytes(d->B, d->N, d->D, d->cell, d->in_dtype == FRNN_F32, path);
  return FRNN_OK;
}

int frnn_plan_str(const frnn_desc* d, int path, char* buf, size_t cap) {
  int rc = validate_desc(d, path);
  if (rc != FRNN_OK) return rc;
  if (!buf || cap == 0) return FRNN_EINVAL;
  Problem p = problem_from_desc(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
  std::string s;
  if (path == FRNN_PATH_FUSED) {
    DevInfo di;
    if (get_devinfo(&di) != FRNN_OK) di = default_devinfo();
    FusedPlan fp;
    rc = plan_fused(p, di, &fp);
    if (rc != FRNN_OK) return rc;
    s = plan_string(p, path, &fp);
  } else {
    s = plan_string(p, path, nullptr);
  }
  std::snprintf(buf, cap, "%s", s.c_str());
  return FRNN_OK;
}

int frnn_fwd(const frnn_desc* d, int path, const void* Wx, const void* R, const void* b, const void* states0,
             void* states, void* last_states, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = validate_desc(d, path);
  if (rc != FRNN_OK) return rc;
  if (d->T > 0 && (!Wx || !R)) return FRNN_EINVAL;
  if (misaligned(Wx) || misaligned(R) || misaligned(b) || misaligned(states0) || misaligned(states) ||
      misaligned(last_states) || misaligned(workspace))
    return FRNN_EINVAL;
  const size_t need = kErrBytes + rec_scratch_bytes(d->B, d->N, d->D, d->cell, d->in_dtype == FRNN_F32, path);
  if (!workspace || workspace_bytes < need) return FRNN_EWORKSPACE;
  Problem p = problem_from_desc(d, Wx, R, b, states0, states, last_states);
  if (path == FRNN_PATH_FUSED) {
    DevInfo di;
    rc = get_devinfo(&di);
    if (rc != FRNN_OK) return rc;
    FusedPlan fp;
    rc = plan_fused(p, di, &fp);
    if (rc != FRNN_OK) return rc;
  } else {
    DevInfo di;
    rc = get_devinfo(&di);
    if (rc != FRNN_OK) return rc;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (launch_fill(workspace, kErrBytes, st) != hipSuccess) return FRNN_EHIP;
  if (d->T == 0) {
    if (last_states) {
      const long long n = (long long)(d->cell == FRNN_CELL_LSTM ? 2 : 1) * d->B * d->N * d->D;
      hipLaunchKernelGGL(copy_init_kernel, dim3((unsigned)std::min<long long>((n + 255) / 256, 4096)), dim3(256), 0, st,
                         states0, d->in_dtype == FRNN_F32 ? 1 : 0, reinterpret_cast<float*>(last_states), n);
      if (hipGetLastError() != hipSuccess) return FRNN_EHIP;
    }
    return FRNN_OK;
  }
  return run_recurrence(p, path, reinterpret_cast<int*>(workspace), reinterpret_cast<char*>(workspace) + kErrBytes, st);
}

int frnn_fwd_noalloc(const frnn_desc* d, int path, const void* Wx, const void* R, const void* b, const void* states0,
                     void* states, void* last_states, void* stream) {
  const int rc = validate_desc(d, path);
  if (rc != FRNN_OK) return rc;
  const size_t need = kErrBytes + rec_scratch_bytes(d->B, d->N, d->D, d->cell, d->in_dtype == FRNN_F32, path);
  if (need > kScratchBytes) return FRNN_EWORKSPACE;
  DevInfo di;
  const int drc = get_devinfo(&di);
  if (drc != FRNN_OK) return drc;
  // frnn_fwd on the array: it clears the error word and fills the exchange words at the start of
  // the call, so nothing of an earlier call's contents is read
  return frnn_fwd(d, path, Wx, R, b, states0, states, last_states, di.scratch, kScratchBytes, stream);
}

int frnn_check(const void* workspace, void* stream) {
  if (!workspace) {  // the error word of frnn_fwd_noalloc's array on the current device
    DevInfo di;
    const int rc = get_devinfo(&di);
    if (rc != FRNN_OK) return rc;
    workspace = di.scratch;
  }
  if (hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return FRNN_EHIP;
  int word = 0;
  if (hipMemcpy(&word, workspace, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return FRNN_EHIP;
  if (word & DEVERR_PLACEMENT) return FRNN_EPLACEMENT;
  if (word & DEVERR_TIMEOUT) return FRNN_ETIMEOUT;
  return FRNN_OK;
}

int frnn_bwd_workspace_bytes(const frnn_desc* d, int path, size_t* bytes) {
  const int rc = validate_desc(d, path);
  if (rc != FRNN_OK) return rc;
  if (!bytes) return FRNN_EINVAL;
  *bytes = kErrBytes + bwd_layout(d->B, d->T, d->N, d->D, d->cell, d->in_dtype == FRNN_F32, path).total;
  return FRNN_OK;
}

int frnn_bwd(const frnn_desc* d, int path, const void* Wx, const void* R, const void* b, const void* states0,
             const void* states, const void* dstates, const void* dlast, void* dWx, void* dR, void* db,
             void* dstates0, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = validate_desc(d, path);
  if (rc != FRNN_OK) return rc;
  if ((long long)((d->B + 15) / 16) * d->N > 65535) return FRNN_EUNSUPPORTED;  // dh kernel grid
  if (d->T > 0 && (!Wx || !R || !states)) return FRNN_EINVAL;
  for (const void* p : {Wx, R, b, states0, states, dstates, dlast, (const void*)dWx, (const void*)dR, (const void*)db,
                        (const void*)dstates0, (const void*)workspace})
    if (misaligned(p)) return FRNN_EINVAL;
  const int f32 = d->in_dtype == FRNN_F32;
  const BwdLayout L = bwd_layout(d->B, d->T, d->N, d->D, d->cell, f32, path);
  if (!workspace || workspace_bytes < kErrBytes + L.total) return FRNN_EWORKSPACE;
  DevInfo di;
  rc = get_devinfo(&di);
  if (rc != FRNN_OK) return rc;
  FusedBwdPlan fbp;
  if (path == FRNN_PATH_FUSED) {
    rc = plan_fused_bwd(d->B, d->N, d->D, d->cell, f32, di, &fbp);
    if (rc != FRNN_OK) return rc;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  trace("[frnn] %s\n", bwd_plan_string(d, path, path == FRNN_PATH_FUSED ? &fbp : nullptr));
  const int B = d->B, T = d->T, N = d->N, D = d->D, G = gates_of(d->cell), S = d->cell == FRNN_CELL_LSTM ? 2 : 1;
  const long long BND = (long long)B * N * D;
  const size_t elt = f32 ? 4 : 2;
  if (launch_fill(workspace, kErrBytes, st) != hipSuccess) return FRNN_EHIP;
  const unsigned sgrid = (unsigned)((BND + 255) / 256);
  if (T == 0) {
    // last_states is the initial state: dstates0 = dlast, and nothing else receives a gradient
    if (dstates0) {
      const long long n = (long long)S * BND;
      if (dlast)
        hipLaunchKernelGGL(copy_init_kernel, dim3((unsigned)std::min<long long>((n + 255) / 256, 4096)), dim3(256), 0, st,
                           dlast, 1, reinterpret_cast<float*>(dstates0), n);
      else if (launch_fill(dstates0, (size_t)n * 4, st) != hipSuccess) return FRNN_EHIP;
    }
    if (dR && launch_fill(dR, (size_t)G * N * D * D * 4, st) != hipSuccess) return FRNN_EHIP;
    if (db && launch_fill(db, (size_t)G * N * D * 4, st) != hipSuccess) return FRNN_EHIP;
    return hipGetLastError() == hipSuccess ? FRNN_OK : FRNN_EHIP;
  }
  const Strides sd = strides_of(d);
  BwdProblem q;
  std::memset(&q, 0, sizeof(q));
  q.B = B; q.T = T; q.N = N; q.D = D; q.cell = d->cell; q.f32 = f32; q.wx_f32 = f32;
  q.Wx = Wx; q.wx_sb = sd.wx_sb; q.wx_st = sd.wx_st;
  q.R = R; q.r_sg = sd.r_sg; q.r_sn = sd.r_sn; q.r_sd = sd.r_sd;
  q.bias = b;
  q.s0_h = states0;
  q.s0_c = (states0 && S == 2) ? reinterpret_cast<const char*>(states0) + (size_t)BND * elt : nullptr;
  q.s0_sb = (long long)N * D;
  const float* stf = reinterpret_cast<const float*>(states);
  q.st_h = stf; q.st_c = S == 2 ? stf + sd.st_ss : nullptr;
  q.st_sb = sd.st_sb; q.st_st = sd.st_st;
  const float* dsf = reinterpret_cast<const float*>(dstates);
  q.ds_h = dsf; q.ds_c = (dsf && S == 2) ? dsf + sd.st_ss : nullptr;
  const float* dlf = reinterpret_cast<const float*>(dlast);
  q.dl_h = dlf; q.dl_c = (dlf && S == 2) ? dlf + BND : nullptr;
  q.last_sb = (long long)N * D;
  q.dWx = reinterpret_cast<float*>(dWx);
  q.dR = reinterpret_cast<float*>(dR); q.dr_sg = sd.r_sg; q.dr_sn = sd.r_sn; q.dr_sd = sd.r_sd;
  q.db = reinterpret_cast<float*>(db);
  q.ds0_h = reinterpret_cast<float*>(dstates0);
  q.ds0_c = (dstates0 && S == 2) ? reinterpret_cast<float*>(dstates0) + BND : nullptr;
  (void)sgrid;
  return run_backward(q, path, fbp, di, reinterpret_cast<char*>(workspace) + kErrBytes, L, st);
}

int frnn_bwd_plan_str(const frnn_desc* d, int path, char* buf, size_t cap) {
  const int rc = validate_desc(d, path);
  if (rc != FRNN_OK) return rc;
  if (!buf || cap == 0) return FRNN_EINVAL;
  FusedBwdPlan fbp;
  if (path == FRNN_PATH_FUSED) {
    DevInfo di;
    if (get_devinfo(&di) != FRNN_OK) di = default_devinfo();
    const int prc = plan_fused_bwd(d->B, d->N, d->D, d->cell, d->in_dtype == FRNN_F32, di, &fbp);
    if (prc != FRNN_OK) return prc;
  }
  std::snprintf(buf, cap, "%s", bwd_plan_string(d, path, path == FRNN_PATH_FUSED ? &fbp : nullptr).c_str());
  return FRNN_OK;
}

static int validate_stack(int L, int dirs, int T, int B, int I, int H, int path) {
  if (L < 1 || T < 0 || B < 1 || I < 1 || H < 1) return FRNN_EINVAL;
  if (dirs != 1 && dirs != 2) return FRNN_EINVAL;
  if (path != FRNN_PATH_ALTERNATING && path != FRNN_PATH_FUSED) return FRNN_EINVAL;
  if ((long long)T * B * 4 * H * dirs > (1LL << 40)) return FRNN_EINVAL;
  if (H % 32 != 0 || H > 1024) return FRNN_EUNSUPPORTED;
  return FRNN_OK;
}

// Workspace of frnn_lstm_stack_fwd after the error word.
struct StackLayout {
  size_t wx, wit, bias, hseq, rcopy, rec, total;
};

static StackLayout stack_layout(int L, int dirs, int T, int B, int I, int H, int path) {
  const size_t G4 = (size_t)4 * H * dirs;  // projected columns of one layer
  StackLayout S;
  size_t q = 0;
  S.wx = q;    q += align256((size_t)T * B * G4 * 4);                        // projected inputs, fp32
  S.wit = q;   q += align256((size_t)std::max(I, dirs * H) * G4 * 2);        // Wi transposed, bf16
  S.bias = q;  q += dirs > 1 ? align256(2 * G4 * 2) : 0;                     // both biases in column order
  S.hseq = q;  q += L > 1 ? align256((size_t)T * B * dirs * H * 4) : 0;      // h sequence for the next layer
  S.rcopy = q; q += dirs > 1 ? align256((size_t)dirs * H * 4 * H * 2) : 0;   // both Wh side by side
  S.rec = q;   q += rec_scratch_bytes(B, dirs, H, FRNN_CELL_LSTM, 0, path);
  S.total = q;
  return S;
}

int frnn_lstm_stack_workspace_bytes(int L, int dirs, int T, int B, int I, int H, int path, size_t* bytes) {
  const int rc = validate_stack(L, dirs, T, B, I, H, path);
  if (rc != FRNN_OK) return rc;
  if (!bytes) return FRNN_EINVAL;
  *bytes = kErrBytes + stack_layout(L, dirs, T, B, I, H, path).total;
  return FRNN_OK;
}

// The layer's projection operand: Bt rows (the projected columns) in the order [gate][direction][unit],
// so that the projection comes out as the head-wise Wx [T][B][G][dirs][H] with one head per
// direction. Row g*dirs*H + n*H + e is column g*H + e of Wi of direction n.
static void stack_transpose_wi(const void* const* Wi, int l, int dirs, int in, int H, uint16_t* wit, hipStream_t st) {
  if (dirs == 1) {
    launch_transpose<uint16_t>(reinterpret_cast<const uint16_t*>(Wi[l]), 4LL * H, in, 4 * H, wit, in, st);
    return;
  }
  for (int n = 0; n < dirs; ++n)
    for (int g = 0; g < 4; ++g)
      launch_transpose<uint16_t>(reinterpret_cast<const uint16_t*>(Wi[l * dirs + n]) + (size_t)g * H, 4LL * H, in, H,
                                 wit + ((size_t)g * dirs * H + (size_t)n * H) * in, in, st);
}

int frnn_lstm_stack_fwd(int L, int dirs, int T, int B, int I, int H, int path, const void* x, const void* const* Wi,
                        const void* const* Wh, const void* const* b_ih, const void* const* b_hh, const void* h0,
                        const void* c0, void* out, void* hn, void* cn, void* workspace, size_t workspace_bytes,
                        void* stream) {
  int rc = validate_stack(L, dirs, T, B, I, H, path);
  if (rc != FRNN_OK) return rc;
  if (!Wi || !Wh) return FRNN_EINVAL;
  if (T > 0 && !x) return FRNN_EINVAL;
  for (int l = 0; l < L * dirs; ++l) {
    if (!Wi[l] || !Wh[l]) return FRNN_EINVAL;
    if (misaligned(Wi[l]) || misaligned(Wh[l])) return FRNN_EINVAL;
    if (b_ih && misaligned(b_ih[l])) return FRNN_EINVAL;
    if (b_hh && misaligned(b_hh[l])) return FRNN_EINVAL;
  }
  if (misaligned(x) || misaligned(h0) || misaligned(c0) || misaligned(out) || misaligned(hn) || misaligned(cn) ||
      misaligned(workspace))
    return FRNN_EINVAL;
  const StackLayout SL = stack_layout(L, dirs, T, B, I, H, path);
  if (!workspace || workspace_bytes < kErrBytes + SL.total) return FRNN_EWORKSPACE;
  DevInfo di;
  rc = get_devinfo(&di);
  if (rc != FRNN_OK) return rc;
  // the per-layer recurrence plan must exist before anything is enqueued
  Problem probe;
  std::memset(&probe, 0, sizeof(probe));
  probe.B = B; probe.T = T; probe.N = dirs; probe.D = H; probe.cell = FRNN_CELL_LSTM; probe.r_f32 = 0; probe.wx_f32 = 1;
  if (path == FRNN_PATH_FUSED) {
    FusedPlan fp;
    rc = plan_fused(probe, di, &fp);
    if (rc != FRNN_OK) return rc;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* base = reinterpret_cast<char*>(workspace) + kErrBytes;
  if (launch_fill(workspace, kErrBytes, st) != hipSuccess) return FRNN_EHIP;
  float* wx = reinterpret_cast<float*>(base + SL.wx);
  uint16_t* wit = reinterpret_cast<uint16_t*>(base + SL.wit);
  uint16_t* biasp = reinterpret_cast<uint16_t*>(base + SL.bias);
  float* hseq = L > 1 ? reinterpret_cast<float*>(base + SL.hseq) : nullptr;
  uint16_t* rcopy = reinterpret_cast<uint16_t*>(base + SL.rcopy);
  void* rws = base + SL.rec;
  const long long LBH = (long long)B * H, G4 = 4LL * H * dirs;
  if (T == 0) {  // the final states are the initial ones
    const long long n = (long long)L * dirs * LBH;
    const unsigned g = (unsigned)std::min<long long>((n + 255) / 256, 4096);
    if (hn) hipLaunchKernelGGL(copy_init_kernel, dim3(g), dim3(256), 0, st, h0, 0, reinterpret_cast<float*>(hn), n);
    if (cn) hipLaunchKernelGGL(copy_init_kernel, dim3(g), dim3(256), 0, st, c0, 0, reinterpret_cast<float*>(cn), n);
    return hipGetLastError() == hipSuccess ? FRNN_OK : FRNN_EHIP;
  }
  for (int l = 0; l < L; ++l) {
    const int in = (l == 0) ? I : dirs * H;
    const long long soff = (long long)l * dirs * LBH;  // this layer's [dirs][B][H] block of h0 / hn
    // projection of the layer's whole input sequence, rows m = t*B + b, columns [gate][direction][unit]
    ProjArgs pa;
    pa.M = T * B; pa.Nc = (int)G4; pa.K = in;
    pa.A = (l == 0) ? x : hseq;
    pa.a_f32 = (l == 0) ? 0 : 1;
    pa.lda = pa.K;
    pa.Bt = wit;
    pa.ldb = pa.K;
    pa.a_z = pa.b_z = pa.c_z = 0;
    pa.a_h = pa.b_h = pa.c_h = 0;
    pa.nt = 0;  // the recurrence reads Wx next: left where its loads find it soonest
    if (dirs == 1) {
      pa.b1 = b_ih ? reinterpret_cast<const uint16_t*>(b_ih[l]) : nullptr;
      pa.b2 = b_hh ? reinterpret_cast<const uint16_t*>(b_hh[l]) : nullptr;
    } else {
      StackBiasArgs ba;
      ba.H = H; ba.dirs = dirs;
      for (int n = 0; n < 2; ++n) {
        ba.bi[n] = b_ih ? reinterpret_cast<const uint16_t*>(b_ih[l * dirs + n]) : nullptr;
        ba.bh[n] = b_hh ? reinterpret_cast<const uint16_t*>(b_hh[l * dirs + n]) : nullptr;
      }
      ba.out = biasp;
      hipLaunchKernelGGL(stack_bias_kernel, dim3((unsigned)((G4 + 255) / 256)), dim3(256), 0, st, ba);
      pa.b1 = biasp;
      pa.b2 = biasp + G4;
    }
    pa.C = wx;
    pa.ldc = G4;
    stack_transpose_wi(Wi, l, dirs, in, H, wit, st);
    const dim3 pgrid(proj_tiles(pa));
    launch_proj(pa, pgrid, st);
    if (hipGetLastError() != hipSuccess) return FRNN_EHIP;
    // recurrence, one head per direction: R[g][n][d][e] = Wh of direction n at [d][g*H + e], read
    // in place for one direction, from a side-by-side copy for two
    Problem p;
    std::memset(&p, 0, sizeof(p));
    p.B = B; p.T = T; p.N = dirs; p.D = H; p.cell = FRNN_CELL_LSTM; p.r_f32 = 0;
    p.Wx = wx; p.wx_f32 = 1; p.wx_sb = G4; p.wx_st = G4 * B;
    if (dirs == 1) {
      p.R = Wh[l]; p.r_sn = 0;
    } else {
      const long long wh = (long long)H * 4 * H;
      for (int n = 0; n < dirs; ++n)
        if (hipMemcpyAsync(rcopy + n * wh, Wh[l * dirs + n], (size_t)wh * 2, hipMemcpyDeviceToDevice, st) != hipSuccess)
          return FRNN_EHIP;
      p.R = rcopy; p.r_sn = wh;
    }
    p.r_sg = H; p.r_sd = 4LL * H;
    p.bias = nullptr;
    p.s0_h = h0 ? reinterpret_cast<const uint16_t*>(h0) + soff : nullptr;
    p.s0_c = c0 ? reinterpret_cast<const uint16_t*>(c0) + soff : nullptr;
    p.s0_f32 = 0; p.s0_sb = H; p.s0_sn = LBH;
    p.out_h = (l == L - 1) ? reinterpret_cast<float*>(out) : hseq;
    p.out_c = nullptr;
    p.out_sb = (long long)dirs * H; p.out_st = (long long)B * dirs * H;
    p.last_h = hn ? reinterpret_cast<float*>(hn) + soff : nullptr;
    p.last_c = cn ? reinterpret_cast<float*>(cn) + soff : nullptr;
    p.last_sb = H; p.last_sn = LBH;
    p.rev_n0 = 1;  // the second direction's head runs backwards in time
    rc = run_recurrence(p, path, reinterpret_cast<int*>(workspace), rws, st);
    if (rc != FRNN_OK) return rc;
  }
  return FRNN_OK;
}

// ----------------------------------------------------------------------------- stack backward
// Workspace of frnn_lstm_stack_bwd (after the error word).
struct StackBwdLayout {
  size_t wx, st, wit, dwx, dx, xt, dwxt, parts, db, wicat, rec, bwd, total;
  BwdLayout bl;
};

// Every layer keeps its projection [T][B][dirs][4H] and its states, h and c each [T][B][dirs*H]
// (direction k at columns k*H), in time order for both directions.
static StackBwdLayout stack_bwd_layout(int L, int dirs, int T, int B, int I, int H, int path) {
  StackBwdLayout S;
  const size_t TB = (size_t)T * B, IH = (size_t)std::max(I, dirs * H), Kp = bwd_kp(T, B);
  const size_t G4 = (size_t)dirs * 4 * H;
  size_t q = 0;
  S.wx = q;    q += align256((size_t)L * TB * G4 * 4);            // every layer's projection, fp32
  S.st = q;    q += align256((size_t)L * 2 * TB * dirs * H * 4);  // every layer's h and c, fp32
  S.wit = q;   q += align256(IH * 4 * H * 2);                     // one direction's Wi transposed
  S.dwx = q;   q += align256(TB * G4 * 4);                        // dWx of the layer at hand
  S.dx = q;    q += align256(2 * TB * IH * 4);                    // dX of the layer above / at hand
  S.xt = q;    q += align256(IH * Kp * 2);                        // the layer's input, transposed, bf16
  S.dwxt = q;  q += align256((size_t)4 * H * Kp * 2);             // one direction's dWx transposed, bf16
  S.parts = q; q += align256((size_t)BWD_DR_PARTS * IH * 4 * H * 4);  // K parts of dWi
  S.db = q;    q += align256((size_t)4 * H * 4);
  S.wicat = q; q += dirs > 1 ? align256(IH * G4 * 2) : 0;         // both directions' Wi side by side along K
  S.rec = q;   q += align256(rec_scratch_bytes(B, 1, H, FRNN_CELL_LSTM, 0, path));  // forward recurrence
  S.bl = bwd_layout(B, T, 1, H, FRNN_CELL_LSTM, 0, path);
  S.bwd = q;   q += align256(S.bl.total);
  S.total = q;
  return S;
}

int frnn_lstm_stack_bwd_workspace_bytes(int L, int dirs, int T, int B, int I, int H, int path, size_t* bytes) {
  const int rc = validate_stack(L, dirs, T, B, I, H, path);
  if (rc != FRNN_OK) return rc;
  if (!bytes) return FRNN_EINVAL;
  *bytes = kErrBytes + stack_bwd_layout(L, dirs, T, B, I, H, path).total;
  return FRNN_OK;
}

int frnn_lstm_stack_bwd(int L, int dirs, int T, int B, int I, int H, int path, const void* x, const void* const* Wi,
                        const void* const* Wh, const void* const* b_ih, const void* const* b_hh, const void* h0,
                        const void* c0, const void* dout, const void* dhn, const void* dcn, void* dx,
                        void* const* dWi, void* const* dWh, void* const* db_ih, void* const* db_hh, void* dh0,
                        void* dc0, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = validate_stack(L, dirs, T, B, I, H, path);
  if (rc != FRNN_OK) return rc;
  if (!Wi || !Wh) return FRNN_EINVAL;
  if (T > 0 && !x) return FRNN_EINVAL;
  const int J = L * dirs;  // (layer, direction) pairs, j = l * dirs + k
  for (int j = 0; j < J; ++j) {
    if (!Wi[j] || !Wh[j] || misaligned(Wi[j]) || misaligned(Wh[j])) return FRNN_EINVAL;
    if ((b_ih && misaligned(b_ih[j])) || (b_hh && misaligned(b_hh[j]))) return FRNN_EINVAL;
    if ((dWi && misaligned(dWi[j])) || (dWh && misaligned(dWh[j])) || (db_ih && misaligned(db_ih[j])) ||
        (db_hh && misaligned(db_hh[j])))
      return FRNN_EINVAL;
  }
  for (const void* p : {x, h0, c0, dout, dhn, dcn, (const void*)dx, (const void*)dh0, (const void*)dc0,
                        (const void*)workspace})
    if (misaligned(p)) return FRNN_EINVAL;
  const StackBwdLayout SL = stack_bwd_layout(L, dirs, T, B, I, H, path);
  if (!workspace || workspace_bytes < kErrBytes + SL.total) return FRNN_EWORKSPACE;
  DevInfo di;
  rc = get_devinfo(&di);
  if (rc != FRNN_OK) return rc;
  // both recurrences' plans must exist before anything is enqueued (every direction of every layer
  // is one head of H units)
  Problem probe;
  std::memset(&probe, 0, sizeof(probe));
  probe.B = B; probe.T = T; probe.N = 1; probe.D = H; probe.cell = FRNN_CELL_LSTM; probe.r_f32 = 0; probe.wx_f32 = 1;
  FusedPlan fp;
  FusedBwdPlan fbp;
  if (path == FRNN_PATH_FUSED) {
    if ((rc = plan_fused(probe, di, &fp)) != FRNN_OK) return rc;
    if ((rc = plan_fused_bwd(B, 1, H, FRNN_CELL_LSTM, 0, di, &fbp)) != FRNN_OK) return rc;
  }
  if ((long long)((B + 15) / 16) > 65535) return FRNN_EUNSUPPORTED;  // dh kernel grid
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* base = reinterpret_cast<char*>(workspace) + kErrBytes;
  if (launch_fill(workspace, kErrBytes, st) != hipSuccess) return FRNN_EHIP;
  const long long TB = (long long)T * B, LBH = (long long)B * H;
  const long long DH = (long long)dirs * H, G4 = 4LL * dirs * H;  // a layer's output and projection widths
  const int Kp = (int)bwd_kp(T, B);
  auto in_of = [&](int l) { return l == 0 ? I : (int)DH; };
  auto fill_out = [&](void* p, size_t bytes) { return p ? launch_fill(p, bytes, st) : hipSuccess; };
  if (T == 0) {  // the final states are the initial ones; nothing else receives a gradient
    for (int j = 0; j < J; ++j) {
      const int in = in_of(j / dirs);
      if ((dWi && fill_out(dWi[j], (size_t)in * 4 * H * 4) != hipSuccess) ||
          (dWh && fill_out(dWh[j], (size_t)H * 4 * H * 4) != hipSuccess) ||
          (db_ih && fill_out(db_ih[j], (size_t)4 * H * 4) != hipSuccess) ||
          (db_hh && fill_out(db_hh[j], (size_t)4 * H * 4) != hipSuccess))
        return FRNN_EHIP;
    }
    const long long n = (long long)J * LBH;
    const unsigned g = (unsigned)std::min<long long>((n + 255) / 256, 4096);
    if (dh0) {
      if (dhn) hipLaunchKernelGGL(copy_init_kernel, dim3(g), dim3(256), 0, st, dhn, 1, reinterpret_cast<float*>(dh0), n);
      else if (fill_out(dh0, (size_t)n * 4) != hipSuccess) return FRNN_EHIP;
    }
    if (dc0) {
      if (dcn) hipLaunchKernelGGL(copy_init_kernel, dim3(g), dim3(256), 0, st, dcn, 1, reinterpret_cast<float*>(dc0), n);
      else if (fill_out(dc0, (size_t)n * 4) != hipSuccess) return FRNN_EHIP;
    }
    return hipGetLastError() == hipSuccess ? FRNN_OK : FRNN_EHIP;
  }
  float* wx_all = reinterpret_cast<float*>(base + SL.wx);
  float* st_all = reinterpret_cast<float*>(base + SL.st);
  uint16_t* wit = reinterpret_cast<uint16_t*>(base + SL.wit);
  float* dwx = reinterpret_cast<float*>(base + SL.dwx);
  const long long IH = std::max<long long>(I, DH);
  float* dxb[2] = {reinterpret_cast<float*>(base + SL.dx), reinterpret_cast<float*>(base + SL.dx) + TB * IH};
  uint16_t* xt = reinterpret_cast<uint16_t*>(base + SL.xt);
  uint16_t* dwxt = reinterpret_cast<uint16_t*>(base + SL.dwxt);
  float* parts = reinterpret_cast<float*>(base + SL.parts);
  float* dbt = reinterpret_cast<float*>(base + SL.db);
  uint16_t* wicat = reinterpret_cast<uint16_t*>(base + SL.wicat);
  int* err = reinterpret_cast<int*>(workspace);
  auto layer_wx = [&](int l) { return wx_all + (size_t)l * TB * G4; };
  auto layer_h = [&](int l) { return st_all + (size_t)l * 2 * TB * DH; };
  auto layer_c = [&](int l) { return layer_h(l) + TB * DH; };
  // 1. the forward again, keeping every layer's projection and states (time-major, time order);
  // direction 1 is a head that runs backwards in time over the same buffers
  for (int l = 0; l < L; ++l) {
    const int in = in_of(l);
    for (int k = 0; k < dirs; ++k) {
      const int j = l * dirs + k;
      ProjArgs pa;
      pa.M = (int)TB; pa.Nc = 4 * H; pa.K = in;
      pa.A = (l == 0) ? x : (const void*)layer_h(l - 1);
      pa.a_f32 = (l == 0) ? 0 : 1;
      pa.lda = in;
      pa.Bt = wit;
      pa.ldb = in;
      pa.a_z = pa.b_z = pa.c_z = 0;
      pa.a_h = pa.b_h = pa.c_h = 0;
      pa.nt = 0;  // the recurrence reads Wx next: left where its loads find it soonest
      pa.b1 = b_ih ? reinterpret_cast<const uint16_t*>(b_ih[j]) : nullptr;
      pa.b2 = b_hh ? reinterpret_cast<const uint16_t*>(b_hh[j]) : nullptr;
      pa.C = layer_wx(l) + (size_t)k * 4 * H;
      pa.ldc = G4;
      launch_transpose<uint16_t>(reinterpret_cast<const uint16_t*>(Wi[j]), 4 * H, in, 4 * H, wit, in, st);
      const dim3 pgrid(proj_tiles(pa));
      launch_proj(pa, pgrid, st);
      if (hipGetLastError() != hipSuccess) return FRNN_EHIP;
      Problem p;
      std::memset(&p, 0, sizeof(p));
      p.B = B; p.T = T; p.N = 1; p.D = H; p.cell = FRNN_CELL_LSTM; p.r_f32 = 0;
      p.Wx = layer_wx(l) + (size_t)k * 4 * H; p.wx_f32 = 1; p.wx_sb = G4; p.wx_st = G4 * B;
      p.R = Wh[j]; p.r_sg = H; p.r_sn = 0; p.r_sd = 4LL * H;
      p.s0_h = h0 ? reinterpret_cast<const uint16_t*>(h0) + j * LBH : nullptr;
      p.s0_c = c0 ? reinterpret_cast<const uint16_t*>(c0) + j * LBH : nullptr;
      p.s0_f32 = 0; p.s0_sb = H; p.s0_sn = H; p.last_sn = H;
      p.rev_n0 = k == 1 ? 0 : 1;  // direction 1: the head runs from step T-1 down
      p.out_h = layer_h(l) + (size_t)k * H; p.out_c = layer_c(l) + (size_t)k * H;
      p.out_sb = DH; p.out_st = DH * B;
      rc = run_recurrence(p, path, err, base + SL.rec, st);
      if (rc != FRNN_OK) return rc;
    }
  }
  // 2. the layers from the top: per direction the recurrence's backward, then the projection's;
  // direction 1 sees its sequences through views that run from step T-1 down (negative time strides)
  for (int l = L - 1; l >= 0; --l) {
    const int in = in_of(l);
    const float* dup = (l == L - 1) ? reinterpret_cast<const float*>(dout) : dxb[(l + 1) & 1];  // [T][B][dirs*H]
    if (dWi) {  // the layer's input, transposed once for both directions' dWi
      if (launch_fill(xt, (size_t)in * Kp * 2, st) != hipSuccess) return FRNN_EHIP;
      const int ty = (int)std::min<long long>((TB + 31) / 32, 65535);
      if (l == 0) launch_transpose<uint16_t>(reinterpret_cast<const uint16_t*>(x), in, (int)TB, in, xt, Kp, st);
      else hipLaunchKernelGGL(transpose_f32_bf16_kernel, dim3((in + 31) / 32, ty), dim3(256), 0, st, layer_h(l - 1),
                              (long long)in, (int)TB, in, xt, (long long)Kp);
    }
    for (int k = 0; k < dirs; ++k) {
      const int j = l * dirs + k;
      const bool rev = k == 1;
      const long long wst = G4 * B, sst = DH * B;  // time strides of Wx / dWx and of the states / their gradients
      const long long w0 = (long long)k * 4 * H + (rev ? (T - 1) * wst : 0);
      const long long s0 = (long long)k * H + (rev ? (T - 1) * sst : 0);
      BwdProblem q;
      std::memset(&q, 0, sizeof(q));
      q.B = B; q.T = T; q.N = 1; q.D = H; q.cell = FRNN_CELL_LSTM; q.f32 = 0; q.wx_f32 = 1;
      q.Wx = layer_wx(l) + w0; q.wx_sb = G4; q.wx_st = rev ? -wst : wst;
      q.R = Wh[j]; q.r_sg = H; q.r_sn = 0; q.r_sd = 4LL * H;
      q.s0_h = h0 ? reinterpret_cast<const uint16_t*>(h0) + j * LBH : nullptr;
      q.s0_c = c0 ? reinterpret_cast<const uint16_t*>(c0) + j * LBH : nullptr;
      q.s0_sb = H;
      q.st_h = layer_h(l) + s0; q.st_c = layer_c(l) + s0; q.st_sb = DH; q.st_st = rev ? -sst : sst;
      q.ds_h = dup ? dup + s0 : nullptr;
      q.dl_h = dhn ? reinterpret_cast<const float*>(dhn) + j * LBH : nullptr;
      q.dl_c = dcn ? reinterpret_cast<const float*>(dcn) + j * LBH : nullptr;
      q.last_sb = H;
      q.dWx = dwx + w0;  // the layout (and views) of Wx
      q.dR = dWh ? reinterpret_cast<float*>(dWh[j]) : nullptr;
      q.dr_sg = H; q.dr_sn = 0; q.dr_sd = 4LL * H;
      q.db = dbt;  // the bias is folded into Wx: db_ih = db_hh = sum of dWx, which the dR GEMM's ones row gives
      q.ds0_h = dh0 ? reinterpret_cast<float*>(dh0) + j * LBH : nullptr;
      q.ds0_c = dc0 ? reinterpret_cast<float*>(dc0) + j * LBH : nullptr;
      rc = run_backward(q, path, fbp, di, base + SL.bwd, SL.bl, st);
      if (rc != FRNN_OK) return rc;
      const long long nb = 4LL * H;
      if (db_ih && db_ih[j])
        hipLaunchKernelGGL(copy_init_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st, dbt, 1,
                           reinterpret_cast<float*>(db_ih[j]), nb);
      if (db_hh && db_hh[j])
        hipLaunchKernelGGL(copy_init_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st, dbt, 1,
                           reinterpret_cast<float*>(db_hh[j]), nb);
      // dWi = X^T . dWx over K = T*B (bf16 operands, K split in parts summed in order); the sum over
      // the steps does not depend on their order, so both directions use the time-order buffers
      if (dWi && dWi[j]) {
        if (launch_fill(dwxt, (size_t)4 * H * Kp * 2, st) != hipSuccess) return FRNN_EHIP;
        const int ty = (int)std::min<long long>((TB + 31) / 32, 65535);
        hipLaunchKernelGGL(transpose_f32_bf16_kernel, dim3((4 * H + 31) / 32, ty), dim3(256), 0, st,
                           dwx + (size_t)k * 4 * H, G4, (int)TB, 4 * H, dwxt, (long long)Kp);
        const int kpart = Kp / BWD_DR_PARTS;
        const long long ptot = (long long)in * 4 * H;
        if (launch_gemm(false, in, 4 * H, kpart, xt, Kp, dwxt, Kp, parts, 4LL * H, st, BWD_DR_PARTS, kpart, kpart, ptot) !=
            hipSuccess)
          return FRNN_EHIP;
        hipLaunchKernelGGL(sum_parts_kernel, dim3((unsigned)std::min<long long>((ptot + 255) / 256, 65536)), dim3(256), 0,
                           st, parts, BWD_DR_PARTS, ptot, reinterpret_cast<float*>(dWi[j]));
      }
    }
    // dX = sum over directions of dWx_k . Wi_k^T: the gradient of the layer below's h sequence, or
    // of x; one GEMM over K = dirs*4H with the directions' Wi side by side
    float* dxo = (l == 0) ? reinterpret_cast<float*>(dx) : dxb[l & 1];
    if (dxo) {
      const void* wcat = Wi[l * dirs];
      if (dirs > 1) {
        for (int k = 0; k < dirs; ++k) {
          const long long n = (long long)in * 4 * H;
          hipLaunchKernelGGL(copy_rows_b16_kernel, dim3((unsigned)std::min<long long>((n + 255) / 256, 65536)), dim3(256),
                             0, st, reinterpret_cast<const uint16_t*>(Wi[l * dirs + k]), 4LL * H, in, 4 * H,
                             wicat + (size_t)k * 4 * H, G4);
        }
        wcat = wicat;
      }
      if (launch_gemm(false, (int)TB, in, (int)G4, dwx, G4, wcat, G4, dxo, in, st, 1, 0, 0, 0, true) != hipSuccess)
        return FRNN_EHIP;
    }
  }
  return hipGetLastError() == hipSuccess ? FRNN_OK : FRNN_EHIP;
}

}  // extern "C"
