// Device-side building blocks shared by the DeltaLog kernels (gfx950, wave64).
//
// One workgroup owns one (sequence, head) tile: the dk x dv fp32 state block
// (64 KiB at 128 x 128), its log entries and its fill counter, so every tile
// has exactly one reader/writer and no atomics are needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "deltalog.h"

namespace dl {

// Register-resident tile geometry (eager kernel): thread (rg, cg) holds rows
// [rg*RPT, rg*RPT + RPT) of the four columns [4cg, 4cg + 4) as RPT float4
// values, read once and written once.  A half wave (32 lanes at dv = 128)
// reads one 512-byte state row per load instruction: four whole 128-byte lines.
template <int DK, int DV>
struct Geo {
  static constexpr int CG = DV / 4;                 // float4 column groups
  static constexpr int RPT = (DK == 128) ? 16 : 8;  // state rows per thread
  static constexpr int RG = DK / RPT;               // row groups
  static constexpr int NT = CG * RG;                // threads per workgroup
  static constexpr int NW = NT / 64;                // waves per workgroup
  static constexpr int LPE = DK / 8;                // lanes per 8-channel group
  static_assert(NT % 64 == 0 && NT >= DK && NT >= DV, "tile geometry");
  static_assert(DK % RPT == 0 && RPT % 4 == 0, "tile geometry");
};

// Streaming tile geometry (decode and fold).  Thread (rg, cg) handles columns
// [4cg, 4cg + 4) of rows (c*RPC + rr)*RG + rg for chunks c < NC and rr < RPC:
// each load instruction of a wave covers 64/CG consecutive whole rows.  Only
// NB chunks (NB*RPC float4 per thread) are in registers at a time, so many
// more tiles fit on a CU than when the whole tile is register-resident.
// In LDS, per-row vectors are stored permuted by perm(i) = (i % RG)*RPT + i/RG,
// which makes the RPC rows of one chunk of one thread four consecutive floats.
// PF_ is the number of log entries whose keys, decays and factors a decode step
// loads before the base (at least the fold stage size).  NT_, when nonzero, sets the
// threads per workgroup; otherwise 256 for tiles of at least 8,192 entries, else 128.
template <int DK, int DV, int PF_ = 0, int NT_ = 0>
struct SGeo {
  static constexpr int NT = NT_ > 0 ? NT_ : (DK * DV >= 8192) ? 256 : 128;  // threads per workgroup
  static constexpr int CG = DV / 4;                          // float4 column groups
  static constexpr int RG = NT / CG;                         // row groups
  static constexpr int RPT = DK / RG;                        // rows per thread
  static constexpr int RPC = 4;                              // rows per chunk
  static constexpr int NC = RPT / RPC;                       // chunks per thread
  static constexpr int NB = NC < 2 ? NC : 2;                 // chunks in flight
  static constexpr int NW = NT / 64;                         // waves per workgroup
  static constexpr int LPE = DK / 8;                         // lanes per log entry (8 channels each)
  static constexpr int NG = NT / LPE;                        // log entries per pass
  static constexpr int MCT = (DK * DV >= 16384) ? 16 : 32;  // fold stage size aimed at
  static constexpr int PF = PF_ > MCT ? PF_ : MCT;           // entries prefetched
  static constexpr int EPF = (PF + NG - 1) / NG;             // entry passes prefetched
  static constexpr int UPF = (PF + RG - 1) / RG;             // log factors prefetched per thread
  // Log entries per fold stage.  A log of up to MC entries is folded from what
  // the read pass already holds: the first stage-size entry passes cover
  // NG*ceil(MCT/NG) entries and the factor prefetch RG*ceil(MCT/RG) entries.
  static constexpr int MC = NG * ((MCT + NG - 1) / NG) < RG * ((MCT + RG - 1) / RG)
                                ? NG * ((MCT + NG - 1) / NG) : RG * ((MCT + RG - 1) / RG);
  static_assert(NT % 64 == 0 && NT >= DK && NT >= DV && 64 % CG == 0, "tile geometry");
  static_assert(RPT % RPC == 0 && NC >= 1, "tile geometry");
  static_assert(MC >= 16 && MC <= 32, "fold stage size");
  __device__ static constexpr int perm(int i) { return (i % RG) * RPT + i / RG; }
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

// Buffer resource over `bytes` bytes at `base` (raw, stride 0).  A load whose
// offset lies beyond the range returns zeros and makes no memory access, which
// masks log slots past the fill without branches (a branch around a load
// makes the compiler wait for it before the base loads can issue).
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ float bload4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void bload8f(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&f)[8]) {
  const uint4 a = bload16(r, off), b = bload16(r, off + 16);
  f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y); f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
  f[4] = __uint_as_float(b.x); f[5] = __uint_as_float(b.y); f[6] = __uint_as_float(b.z); f[7] = __uint_as_float(b.w);
}
__device__ __forceinline__ float4 bload_factor4(__amdgpu_buffer_rsrc_t r, uint32_t off, float) {
  const uint4 v = bload16(r, off);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
__device__ __forceinline__ float4 bload_factor4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint16_t) {
  return widen4(bload8(r, off));
}

// Stores of results that nothing later in the same launch reads (outputs, log
// appends, folded bases), non-temporal (the nt policy streams the line out of
// the cache rather than keeping it), through a buffer resource at a
// workgroup-uniform base; `off` is the lane's byte offset.  Measured on MI355X:
// 1.7 % less time per decode step with the pool larger than the last-level cache.
constexpr int kStreamStore = 2;  // buffer-store cache-policy bits: nt
__device__ __forceinline__ void store_res(void* base, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), make_rsrc(base, 0x7fffffff), off, 0, kStreamStore);
}
__device__ __forceinline__ void store_res(void* base, uint32_t off, uint2 v) {
  typedef uint32_t u2v __attribute__((ext_vector_type(2)));
  const u2v x = {v.x, v.y};
  __builtin_amdgcn_raw_buffer_store_b64(x, make_rsrc(base, 0x7fffffff), off, 0, kStreamStore);
}
__device__ __forceinline__ void store_res(void* base, uint32_t off, uint4 v) {
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  const u4v x = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(x, make_rsrc(base, 0x7fffffff), off, 0, kStreamStore);
}
__device__ __forceinline__ void store_res(void* base, uint32_t off, float4 v) {
  store_res(base, off, make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                                  __float_as_uint(v.w)));
}

// fp32 -> bf16 bits, round to nearest, ties to even (finite values).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Access to the base in groups of four consecutive elements of a row: fp32, or
// bf16 (the low-bit base, rounded to nearest even when written).
template <bool BF>
struct BaseIO;
template <>
struct BaseIO<false> {
  using T = float;
  __device__ static T* tile(void* base, size_t elem) { return static_cast<T*>(base) + elem; }
  __device__ static float4 load(const T* t, size_t g) { return reinterpret_cast<const float4*>(t)[g]; }
  __device__ static void store(T* t, size_t g, float4 x) { store_res(t, (uint32_t)(g * 16), x); }
};
template <>
struct BaseIO<true> {
  using T = uint16_t;
  __device__ static T* tile(void* base, size_t elem) { return static_cast<T*>(base) + elem; }
  __device__ static float4 load(const T* t, size_t g) { return widen4(reinterpret_cast<const uint2*>(t)[g]); }
  __device__ static void store(T* t, size_t g, float4 x) {
    store_res(t, (uint32_t)(g * 8), make_uint2(f32_to_bf16_rne(x.x) | (f32_to_bf16_rne(x.y) << 16),
                                               f32_to_bf16_rne(x.z) | (f32_to_bf16_rne(x.w) << 16)));
  }
};

__device__ __forceinline__ float step_log2_decay(float d) {
  return fmaxf(log2f(d), kMinLog2Decay);
}

// x as held by the lane that DPP control CTRL selects within this lane's row of 16.
template <int CTRL>
__device__ __forceinline__ float dpp_from(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// x as held by lane l ^ 16 (ROWS == 16) or l ^ 32 (ROWS == 32): one v_permlane16_swap or
// v_permlane32_swap of x with itself, which leaves the partner's value in one of its two
// results, and a select.
template <int ROWS>
__device__ __forceinline__ float lane_xor_rows(float x) {
  const uint32_t u = __float_as_uint(x);
  const int lane = __lane_id();
  if constexpr (ROWS == 16) {
    // results: rows (0, 0, 2, 2) and (1, 1, 3, 3) of x
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
  } else {
    // results: halves (0, 0) and (1, 1) of x
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
  }
}

// Sum over groups of WIDTH consecutive lanes (a power of two <= 64), received by every
// lane of the group.  Each step adds the value of a partner lane whose own partner is this
// lane (lane ^ 1 and lane ^ 2 by quad permutations, then the mirror images within 8 and
// within 16 lanes by DPP, then lane ^ 16 and lane ^ 32 by permlane swaps), so the two
// lanes of a pair add the same two numbers and every lane of a group ends with the same
// bits.
template <int WIDTH>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(WIDTH >= 1 && WIDTH <= 64 && (WIDTH & (WIDTH - 1)) == 0, "lane groups");
  if constexpr (WIDTH >= 2) x += dpp_from<0xB1>(x);   // quad_perm(1, 0, 3, 2): lane ^ 1
  if constexpr (WIDTH >= 4) x += dpp_from<0x4E>(x);   // quad_perm(2, 3, 0, 1): lane ^ 2
  if constexpr (WIDTH >= 8) x += dpp_from<0x141>(x);  // row_half_mirror: 7 - lane within 8
  if constexpr (WIDTH >= 16) x += dpp_from<0x140>(x); // row_mirror: 15 - lane within 16
  if constexpr (WIDTH >= 32) x += lane_xor_rows<16>(x);
  if constexpr (WIDTH >= 64) x += lane_xor_rows<32>(x);
  return x;
}

// Sum the lanes of a wave that hold the same column group: lanes cg, cg+CG, cg+2CG, ...
// (CG = 16 or 32: partners lane ^ 16 and lane ^ 32, by permlane swaps).
template <int CG>
__device__ __forceinline__ float colgroup_sum(float x) {
  static_assert(CG == 16 || CG == 32 || CG == 64, "column groups of 16 or 32 lanes");
  if constexpr (CG <= 16) x += lane_xor_rows<16>(x);
  if constexpr (CG <= 32) x += lane_xor_rows<32>(x);
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
  void* base;  // fp32 or bf16 [tiles][dk][dv] (BaseIO)
  uint16_t* log_k;
  void* log_u;
  float* log_c;
  int32_t* fill;
  int heads;
  int L;
  int tiles;  // batch * heads
};

// Arguments of the prefill kernels: a prompt of `tokens` rows per sequence,
// [batch][tokens][heads][d] for q, k, v, out (and KDA/RWKV6 decay) and
// [batch][tokens][heads] for beta, eta (and GDN decay).
struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* decay;
  const float* beta;
  const float* eta;
  const float* bonus;  // RWKV6: [heads][dk]
  float* out;
  float eps;
  int tokens;
};

struct StepArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* decay;
  const float* beta;
  const float* bonus;
  float* out;
  const float* eta;  // Kaczmarz step size: beta = eta / (||k||^2 + eps) when set
  float eps;
};

}  // namespace dl
