// Device-side helpers shared by the gfx950 kernels: vector types, conversions, gate functions,
// hardware ids. Written for CDNA4 (wave64) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace frnn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));

enum { CELL_LSTM = 0, CELL_ELMAN = 1, CELL_GRU = 2 };

// Gates of a cell as they are stored in Wx, R and b (LSTM i, f, z, o; GRU r, z, n; Elman one).
__host__ __device__ constexpr int cell_gates(int cell) { return cell == CELL_LSTM ? 4 : cell == CELL_GRU ? 3 : 1; }
// Rows a hidden unit takes in a 16-row MFMA tile of R^T: the LSTM and the GRU put one unit's gates
// in four consecutive rows (the GRU's fourth row is zero), so that one lane of the result holds
// all of them; an Elman tile holds sixteen units.
__host__ __device__ constexpr int cell_slots(int cell) { return cell == CELL_ELMAN ? 1 : 4; }

// Bits of the device error word kept at the start of every workspace.
enum { DEVERR_TIMEOUT = 1, DEVERR_PLACEMENT = 2 };

__device__ __forceinline__ float bf2f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float ld_f(const void* p, long long i, bool is_f32) {
  return is_f32 ? reinterpret_cast<const float*>(p)[i] : bf2f(reinterpret_cast<const uint16_t*>(p)[i]);
}

// Logistic sigmoid 1 / (1 + e^-x), with e^-x evaluated as 2^(-x * log2(e)) on the hardware
// exponential and the reciprocal on the hardware reciprocal. Saturates to exactly 0 / 1 for large
// |x| (2^+inf = inf, 1/inf = 0) and propagates NaN.
__device__ __forceinline__ float sigmoid_f(float x) {
  const float e = __builtin_amdgcn_exp2f(x * -1.44269504088896340736f);
  return __builtin_amdgcn_rcpf(1.0f + e);
}

// tanh(x) = 2 * sigmoid(2x) - 1. Absolute error stays at the few-1e-7 level, which is what the
// state update needs (the states are compared in absolute terms).
__device__ __forceinline__ float tanh_f(float x) { return 2.0f * sigmoid_f(2.0f * x) - 1.0f; }

// Hardware id of the accelerator die (XCC) this wave runs on.
__device__ __forceinline__ int xcc_id() {
  return (int)(__builtin_amdgcn_s_getreg((20) | (0 << 6) | (15 << 11)) & 0xFu);
}

// Position of this workgroup in a die-local launch, as (slot * n_xcd + die): the die is the index in
// xcc_of (four bits per die) of the hardware XCC the workgroup runs on, the slot its rank among the
// launch's workgroups on that die, drawn from the die's counter in ctr (which the host fills with
// 0xFFFF before the launch). Groups are then formed from the workgroups that really share a die,
// whatever order the hardware deals them in. -1 (after recording a placement error) for an XCC
// missing from xcc_of or a die that received more than `slots` workgroups. Every thread of the
// workgroup calls it: it contains a workgroup barrier.
__device__ __forceinline__ int die_position(uint32_t xcc_of, int n_xcd, uint32_t* ctr, int slots, int* err) {
  __shared__ int s_pos;
  if (threadIdx.x == 0) {
    const int x = xcc_id();
    int d = -1;
    for (int k = 0; k < n_xcd; ++k)
      if ((int)((xcc_of >> (4 * k)) & 0xFu) == x) d = k;
    int pos = -1;
    if (d >= 0) {
      const int s = (int)(atomicAdd(ctr + d, 1u) - 0xFFFFu);
      if (s >= 0 && s < slots) pos = s * n_xcd + d;
    }
    if (pos < 0) atomicOr(err, DEVERR_PLACEMENT);
    s_pos = pos;
  }
  __syncthreads();
  return s_pos;
}

// Pack the high halves of two 32-bit exchange words (bf16 << 16 | tag) into one bf16 pair.
__device__ __forceinline__ uint32_t pack_hi(uint32_t lo_word, uint32_t hi_word) {
  return __builtin_amdgcn_perm(hi_word, lo_word, 0x07060302u);
}

__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace frnn
