// Shared device helpers and host glue of the WitCert HIP library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/witcert.h"

namespace wc {

// ---------------------------------------------------------------- host glue
void set_error(const char* fmt, ...);
int check_launch(const char* what);

// ---------------------------------------------------------------- dither
// pcg hash of Jarzynski and Olano, "Hash Functions for GPU Rendering",
// JCGT 9(3), 2020: one LCG step followed by the RXS-M-XS output permutation.
constexpr uint32_t kPcgMul = 747796405u, kPcgInc = 2891336453u;
// the output permutation of one LCG state
__host__ __device__ __forceinline__ uint32_t pcg_out(uint32_t state) {
  uint32_t word = ((state >> ((state >> 28u) + 4u)) ^ state) * 277803737u;
  return (word >> 22u) ^ word;
}
__host__ __device__ __forceinline__ uint32_t pcg(uint32_t v) { return pcg_out(v * kPcgMul + kPcgInc); }
// The same permutation in six VALU instructions instead of eight: the shift
// s >> ((s >> 28) + 4) is (s >> 4) >> (s >> 28), and s >> 28 is byte 3 of
// s >> 4, which an SDWA operand select of the shift amount reads directly.
__device__ __forceinline__ uint32_t pcg_out_sdwa(uint32_t state) {
  const uint32_t u = state >> 4u;
  uint32_t r;
  asm("v_lshrrev_b32_sdwa %0, %1, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3 src1_sel:DWORD"
      : "=v"(r)
      : "v"(u));
  const uint32_t word = (r ^ state) * 277803737u;
  return (word >> 22u) ^ word;
}
// The LCG step is linear: the state of counter v + i is the state of v plus
// i * kPcgMul, so runs of consecutive counters need one multiply in all.

// 32-bit key of the dither of one (sequence, layer, KV head), chained from
// the 64-bit sequence seed, the layer and the KV head.
__host__ __device__ __forceinline__ uint32_t stream_key(uint64_t seed, uint32_t layer, uint32_t kv_head) {
  uint32_t k = pcg((uint32_t)(seed >> 32));
  k = pcg(k ^ (uint32_t)seed);
  k = pcg(k ^ layer);
  return pcg(k ^ kv_head);
}

// One draw per (token t, channel c), shared by the key and the value there:
// word j = 64 t + c/2 (low half = even channel), k = 16-bit half of
// pcg(key + j), xi = k * 2^-16 - 1/2.  INT8 codes are stored as offset binary
// (code + 128).

// ---------------------------------------------------------------- numerics
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Exact-rounding fp32 ops (the write path must agree bit for bit with a
// float32 replay; the library is built with -ffp-contract=off as well).
__device__ __forceinline__ float mul_rn(float a, float b) { return __fmul_rn(a, b); }
__device__ __forceinline__ float add_rn(float a, float b) { return __fadd_rn(a, b); }
__device__ __forceinline__ float div_rn(float a, float b) { return __fdiv_rn(a, b); }

// Witness rounding guard.  With u = 2^-24: each residual is one rounding of
// the exact r (relative u), its square enters a sum of nonnegative terms whose
// longest chain has at most 12 roundings, and the square root adds at most 2u,
// so the float32 norm is >= (1 - 9u) of the exact one; the guard 1 + 16u (one
// more rounding on the product) keeps the stored value above it.
constexpr float kWitnessGuard = 1.0f + 9.5367431640625e-07f;   // 1 + 2^-20

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// All-reduce over the 16 lanes of a DPP row: rotations by 8 and 4 within
// the row, then the quad swaps; VALU only, no LDS round trip.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kRowRor8 = 0x128, kRowRor4 = 0x124, kQuadSwap2 = 0x4E, kQuadSwap1 = 0xB1;
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<kRowRor8>(v));
  v = fmaxf(v, dpp_f<kRowRor4>(v));
  v = fmaxf(v, dpp_f<kQuadSwap2>(v));
  return fmaxf(v, dpp_f<kQuadSwap1>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<kRowRor8>(v);
  v += dpp_f<kRowRor4>(v);
  v += dpp_f<kQuadSwap2>(v);
  return v + dpp_f<kQuadSwap1>(v);
}

}  // namespace wc
