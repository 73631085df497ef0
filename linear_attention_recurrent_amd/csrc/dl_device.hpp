// Device-side building blocks shared by the DeltaLog kernels (gfx950, wave64).
//
// Tile geometry.  One workgroup owns one (sequence, head) tile: the dk x dv
// fp32 state block (64 KiB at 128 x 128), its log entries and its fill
// counter, so every tile has exactly one reader/writer and no atomics are
// needed.  Thread (rg, cg) holds rows [rg*RPT, rg*RPT + RPT) of the four
// columns [4cg, 4cg + 4) in registers as RPT float4 values.  A half wave (32
// lanes at dv = 128) therefore reads one 512-byte state row per load
// instruction: four whole 128-byte lines, fully coalesced.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/deltalog.h"

namespace dl {

template <int DK, int DV>
struct Geo {
  static constexpr int CG = DV / 4;                 // float4 column groups
  static constexpr int RPT = (DK == 128) ? 16 : 8;  // state rows per thread
  static constexpr int RG = DK / RPT;               // row groups
  static constexpr int NT = CG * RG;                // threads per workgroup
  static constexpr int NW = NT / 64;                // waves per workgroup
  static constexpr int RG_PER_WAVE = 64 / CG;       // row groups sharing one wave
  static constexpr int LPE = DK / 8;                // lanes per log entry (8 channels each)
  static constexpr int NG = NT / LPE;               // log entries per pass
  static constexpr int UPF = 2;                     // log factors prefetched per thread
  static constexpr int MC = 16;                     // log entries staged per merge chunk
  static_assert(NT % 64 == 0 && NT >= DK && NT >= DV, "tile geometry");
  static_assert(DK % RPT == 0 && RPT % 4 == 0, "tile geometry");
};

// Lowest per-step log2 decay: 2^-126 is the smallest normal float, so a zero
// or denormal decay still gives finite differences of cumulative decays.
constexpr float kMinLog2Decay = -126.0f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Unpack 8 bf16 values held in a uint4 (little-endian: element 0 in the low half of .x).
__device__ __forceinline__ void unpack8(const uint4 w, float (&f)[8]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(ws[i] << 16);
    f[2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ void load8(const float* src, float (&f)[8]) {
  const float4 a = reinterpret_cast<const float4*>(src)[0];
  const float4 b = reinterpret_cast<const float4*>(src)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// Four consecutive factors as fp32: either already fp32, or four bf16 patterns.
__device__ __forceinline__ float4 widen4(const float4 x) { return x; }
__device__ __forceinline__ float4 widen4(const uint2 w) {
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
}

__device__ __forceinline__ float step_log2_decay(float d) {
  return fmaxf(log2f(d), kMinLog2Decay);
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = WIDTH / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Sum the lanes of a wave that hold the same column group: lanes cg, cg+CG, cg+2CG, ...
template <int CG>
__device__ __forceinline__ float colgroup_sum(float x) {
#pragma unroll
  for (int off = CG; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ float4 f4_fma(float s, const float4 a, const float4 c) {
  return make_float4(fmaf(s, a.x, c.x), fmaf(s, a.y, c.y), fmaf(s, a.z, c.z), fmaf(s, a.w, c.w));
}

__device__ __forceinline__ float4 f4_mul(const float4 a, float s) {
  return make_float4(a.x * s, a.y * s, a.z * s, a.w * s);
}

// Arguments of the decode and merge kernels.
struct PoolArgs {
  float* base;
  uint16_t* log_k;
  void* log_u;
  float* log_c;
  int32_t* fill;
  int heads;
  int L;
};

struct StepArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* decay;
  const float* beta;
  const float* bonus;
  float* out;
};

}  // namespace dl
