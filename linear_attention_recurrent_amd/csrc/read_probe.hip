// Memory-rate probes for the benchmark (libdlprobe.so, not part of the decode library).
//
// One workgroup of 256 threads per tile moves the tile's bytes once and keeps
// nothing, with every load issued before any is used: the access shapes of the
// decode and eager steps with no arithmetic around them.  Timed over the very
// pools the decode step uses, they give the rate the memory system delivers for
// each shape, launch size and cache state, in the same run as the kernels:
//   read          the tile (the decode step's base read)
//   read + log    the tile, then `log_bytes` more from the tile's own region of a
//                 second array (the base read plus the log entries a step reads)
//   read + write  the tile, written back in place (the eager step's traffic)
//   stream        the same bytes as 16 KiB units read by persistent workgroups (one
//                 per CU) through four LDS buffers, each unit loaded straight into
//                 LDS: three units in flight per CU, no registers held
//   owned stream  persistent workgroups (one per CU) that own whole 128 x 128 fp32
//                 tiles, as a decode step does: one wave streams each tile's four
//                 16 KiB units straight into a ring of eight LDS buffers, three
//                 ahead of the one read, and four waves form the tile's column sums
//                 from LDS (a decode step's base matvec with nothing around it); or,
//                 for comparison, the same kernel taking the pool's units in the
//                 stream order above
//   quarter split one workgroup per 16 KiB quarter (32 rows) of a 128 x 128 fp32 tile,
//                 the quarters of a tile in consecutive workgroups (so that all of
//                 them sweep one contiguous region): partial column sums of the
//                 quarter, stored; optionally added up across the four workgroups
//                 of the tile by the last to arrive, behind agent-scope fences
// Loaded values feed a sum that is stored only if it equals a value no sum of
// finite inputs hits in practice, so the loads cannot be dropped; the write-back
// scales by 1 - 2^-24 rounded, so it rewrites every value (the stored values change
// by at most one unit in their last place per launch).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kMaxLogPieces = 16;  // 16-byte pieces of log per thread: up to 64 KiB per tile

template <int FPT, int MODE>  // MODE 0: read; 1: read + log; 2: read + write
__global__ void __launch_bounds__(kThreads) tile_probe_kernel(float4* __restrict__ src, const float4* __restrict__ log,
                                                              int log_pieces, int log_stride_pieces, float* sink) {
  const size_t base = (size_t)blockIdx.x * kThreads * FPT;
  float4 v[FPT];
#pragma unroll
  for (int i = 0; i < FPT; ++i) v[i] = src[base + (size_t)i * kThreads + threadIdx.x];
  float4 w[MODE == 1 ? kMaxLogPieces : 1];
  if constexpr (MODE == 1) {
    const size_t lb = (size_t)blockIdx.x * log_stride_pieces;
#pragma unroll
    for (int i = 0; i < kMaxLogPieces; ++i) {
      const int piece = i * kThreads + threadIdx.x;
      w[i] = piece < log_pieces ? log[lb + piece] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  if constexpr (MODE == 2) {
    constexpr float kScale = 1.0f - 5.9604645e-8f;
#pragma unroll
    for (int i = 0; i < FPT; ++i) {
      const float4 x = v[i];
      src[base + (size_t)i * kThreads + threadIdx.x] = make_float4(x.x * kScale, x.y * kScale, x.z * kScale, x.w * kScale);
    }
  } else {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < FPT; ++i) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    if constexpr (MODE == 1) {
#pragma unroll
      for (int i = 0; i < kMaxLogPieces; ++i) s += (w[i].x + w[i].y) + (w[i].z + w[i].w);
    }
    if (s == 1.2345678e30f) sink[blockIdx.x & 255] = s;
  }
}

template <int MODE>
int launch(void* src, const void* log, int log_pieces, int log_stride_pieces, int tile_bytes, int tiles, void* sink,
           hipStream_t st) {
  float4* s = static_cast<float4*>(src);
  const float4* l = static_cast<const float4*>(log);
  float* k = static_cast<float*>(sink);
  switch (tile_bytes) {
    case 16384: tile_probe_kernel<4, MODE><<<tiles, kThreads, 0, st>>>(s, l, log_pieces, log_stride_pieces, k); break;
    case 32768: tile_probe_kernel<8, MODE><<<tiles, kThreads, 0, st>>>(s, l, log_pieces, log_stride_pieces, k); break;
    case 65536: tile_probe_kernel<16, MODE><<<tiles, kThreads, 0, st>>>(s, l, log_pieces, log_stride_pieces, k); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

typedef __attribute__((address_space(3))) void lds_void;

// Four 16-byte LDS reads at byte offsets a, a + S, a + 2S, a + 3S, waited for inside
// the same asm block (the compiler would otherwise wait for every outstanding
// direct-to-LDS load before any LDS read it issues, emptying the pipeline).
#define PROBE_LDS_READ4(r0, r1, r2, r3, a, S)                                                          \
  asm volatile("ds_read_b128 %0, %4\n ds_read_b128 %1, %4 offset:%5\n ds_read_b128 %2, %4 offset:%6\n" \
               " ds_read_b128 %3, %4 offset:%7\n s_waitcnt lgkmcnt(0)"                                 \
               : "=v"(r0), "=v"(r1), "=v"(r2), "=v"(r3)                                                \
               : "v"(a), "n"(S), "n"(2 * (S)), "n"(3 * (S)))

constexpr int kStreamThreads = 256;
constexpr int kStreamBufs = 4;                      // three units in flight while one is read
constexpr int kStreamUnitF4 = 4 * kStreamThreads;  // 16 KiB: four 16-byte pieces per thread

__global__ void __launch_bounds__(kStreamThreads) tile_stream_kernel(const float4* __restrict__ src, int units,
                                                                     float* sink) {
  __shared__ float4 buf[kStreamBufs][kStreamUnitF4];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int G = gridDim.x, wg = blockIdx.x;
  auto issue = [&](int u, int b) {  // 4 x 16 bytes per thread, 1 KiB per wave instruction
    const float4* g = src + (size_t)u * kStreamUnitF4 + tid;
#pragma unroll
    for (int f = 0; f < 4; ++f)
      __builtin_amdgcn_global_load_lds(g + f * kStreamThreads,
                                       (lds_void*)(&buf[b][f * kStreamThreads + wave * 64]), 16, 0, 0);
  };
#pragma unroll
  for (int k = 0; k < kStreamBufs - 1; ++k)
    if (wg + k * G < units) issue(wg + k * G, k);
  float s = 0.f;
  int b = 0;
  for (int u = wg; u < units; u += G) {
    const int un = u + (kStreamBufs - 1) * G;
    if (un < units) {
      issue(un, (b + kStreamBufs - 1) % kStreamBufs);
      asm volatile("s_waitcnt vmcnt(12)" ::: "memory");  // this unit's 4 loads have landed, 12 still in flight
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __builtin_amdgcn_s_barrier();
    const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&buf[b][tid]));
    float4 x0, x1, x2, x3;
    PROBE_LDS_READ4(x0, x1, x2, x3, a, kStreamThreads * 16);
    s += (x0.x + x1.y) + (x2.z + x3.w);
    __builtin_amdgcn_s_barrier();  // every wave is done with this buffer before it is refilled
    b = (b + 1) % kStreamBufs;
  }
  if (s == 1.2345678e30f) sink[wg & 255] = s;
}

// ---------------------------------------------------------------- owned stream
// Workgroup of 320 threads: wave 0 only issues direct-to-LDS loads, from inline asm so
// that the compiler neither counts them nor waits for them (it would otherwise wait for
// every such load in flight before any LDS read); its own s_waitcnt before each barrier
// holds the units issued after the one about to be read (16 instructions of 1 KiB per
// unit).  Waves 1..4 never load from global memory: every LDS read of theirs follows a
// barrier that wave 0 reaches only once the unit has landed.  One barrier per unit.
// Column sums:  out[t][c] = sum_r B_t[r][c] y(t, r),  y(t, r) = 1 + ((131 t + r) mod 7) / 8.
// ORDER 0: workgroup w owns tiles w, w + G, ... (units in order).  ORDER 1: workgroup w
// reads units w, w + G, w + 2G, ... of the pool and sums each run of four as "tile"
// w + i G with unit j of the run at rows 32 j..32 j + 31 (needs G | tiles).  ORDER 2: as
// 0, each tile's units read starting at unit w mod 4.  ORDER 3: workgroup w owns the
// contiguous tiles w P .. w P + P - 1, P = ceil(tiles / G).
constexpr int kOwnThreads = 320;
constexpr int kOwnRing = 8;
constexpr int kOwnAhead = 3;         // units in flight beyond the one awaited
constexpr int kOwnUnitF4 = 1024;     // 16 KiB
constexpr int kOwnUnitsPerTile = 4;  // 128 x 128 fp32

__device__ __forceinline__ float own_weight(int t, int r) { return 1.f + (float)((t * 131 + r) % 7) * 0.125f; }

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is written by the asm and declared clobbered
// Sixteen 1 KiB direct-to-LDS loads: lane l of load f copies the 16 bytes at g + f * 64 + l
// (float4 units) to LDS byte lds + f * 1024 + 16 l (the hardware adds 16 l to m0).
__device__ __forceinline__ void own_issue_unit(const float4* g, uint32_t lds) {
#pragma unroll
  for (int f = 0; f < 16; f += 4)
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, off\n\t"
        "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %5, off\n\t"
        "s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %6, off\n\t"
        "s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %7, off" ::"s"(lds + f * 1024),
        "s"(lds + (f + 1) * 1024), "s"(lds + (f + 2) * 1024), "s"(lds + (f + 3) * 1024), "v"(g + f * 64),
        "v"(g + (f + 1) * 64), "v"(g + (f + 2) * 64), "v"(g + (f + 3) * 64)
        : "memory", "m0");
}
#pragma clang diagnostic pop

template <int ORDER>
__global__ void __launch_bounds__(kOwnThreads) owned_stream_kernel(const float4* __restrict__ src, int tiles,
                                                                   float* __restrict__ out) {
  __shared__ float4 ring[kOwnRing][kOwnUnitF4];
  __shared__ float red[4][128];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = gridDim.x, wg = blockIdx.x;
  const int per = (tiles + G - 1) / G;
  const int ntile = ORDER == 3 ? max(0, min(per, tiles - wg * per)) : tiles > wg ? (tiles - wg + G - 1) / G : 0;
  const int K = ntile * kOwnUnitsPerTile;  // units this workgroup reads, in phase order
  auto tile_of = [&](int i) { return ORDER == 3 ? wg * per + i : wg + i * G; };
  auto unit_of = [&](int k) {              // the unit of its tile read in phase k
    return ORDER == 2 ? (k + wg) % kOwnUnitsPerTile : k % kOwnUnitsPerTile;
  };
  auto unit_at = [&](int k) -> size_t {    // pool index of the unit read in phase k
    if (ORDER == 1) return (size_t)wg + (size_t)k * G;
    return (size_t)tile_of(k / kOwnUnitsPerTile) * kOwnUnitsPerTile + unit_of(k);
  };
  auto issue = [&](int k) {
    own_issue_unit(src + unit_at(k) * kOwnUnitF4 + lane, (uint32_t)(uintptr_t)&ring[k % kOwnRing][0]);
  };
  int issued = 0;
  if (wave == 0) {
    issued = K < kOwnAhead ? K : kOwnAhead;
    for (int k = 0; k < issued; ++k) issue(k);
  }
  // consumer wave c = wave - 1, lane (h, q): rows 8c + 4h + i (i < 4) of each unit, columns 4q..4q+3
  const int c = wave - 1, h = lane >> 5, q = lane & 31;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int ph = 0; ph <= K; ++ph) {  // phase K only finishes the last tile
    if (wave == 0 && ph < K) {
      const int want = ph + kOwnAhead + 1 < K ? ph + kOwnAhead + 1 : K;
      while (issued < want) issue(issued++);  // unit k takes the slot of unit k - 8, read 5 or more phases ago
      const int after = issued - ph - 1;      // units issued after unit ph
      if (after >= 3) asm volatile("s_waitcnt vmcnt(48)" ::: "memory");
      else if (after == 2) asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
      else if (after == 1) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (wave == 0) continue;
    const int i = ph / kOwnUnitsPerTile, u = ph % kOwnUnitsPerTile;
    if (u == 0 && i > 0 && lane < 32) {  // tile i - 1, columns 32c..32c+31
      const int col = 32 * c + lane;
      const float sum = (red[0][col] + red[1][col]) + (red[2][col] + red[3][col]);
      __builtin_nontemporal_store(sum, out + (size_t)tile_of(i - 1) * 128 + col);
    }
    if (ph == K) continue;
    const int t = tile_of(i), ur = ORDER == 1 ? u : unit_of(ph);
    const float4* sl = &ring[ph % kOwnRing][0];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 8 * c + 4 * h + r;
      const float4 x = sl[row * 32 + q];
      const float y = own_weight(t, 32 * ur + row);
      acc.x = fmaf(y, x.x, acc.x);
      acc.y = fmaf(y, x.y, acc.y);
      acc.z = fmaf(y, x.z, acc.z);
      acc.w = fmaf(y, x.w, acc.w);
    }
    if (u == kOwnUnitsPerTile - 1) {  // red is read in the next phase and rewritten four phases later
      acc.x += __shfl_xor(acc.x, 32);
      acc.y += __shfl_xor(acc.y, 32);
      acc.z += __shfl_xor(acc.z, 32);
      acc.w += __shfl_xor(acc.w, 32);
      if (h == 0) *reinterpret_cast<float4*>(&red[c][4 * q]) = acc;
      acc = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// ---------------------------------------------------------------- quarter split
// Workgroup b (256 threads) reads quarter q = b mod 4 of tile t = b / 4 (rows 32 q ..
// 32 q + 31), forms its column sums with two row weights,
//   part[b][c] = sum_r B_t[r][c] own_weight(t, r),  part[b][128 + c] = sum_r B_t[r][c] qs_weight(t, r),
// and stores them.  With EXCHANGE, every thread then fences at agent scope (release),
// thread 0 adds 1 to cnt[t], and the workgroup that finds 3 there fences again (acquire),
// writes out[t] = the sum of the tile's four partials and sets cnt[t] back to 0: a tile's
// column sums finished inside the launch, correct under the HIP memory model (on this chip
// an agent-scope fence writes the L2 back and invalidates it).  No workgroup waits for
// another.
__device__ __forceinline__ float qs_weight(int t, int r) { return 0.5f + (float)((t * 17 + r) % 5) * 0.25f; }

template <bool EXCHANGE>
__global__ void __launch_bounds__(256) quarter_split_kernel(const float4* __restrict__ src, float* __restrict__ part,
                                                            unsigned* __restrict__ cnt, float* __restrict__ out) {
  __shared__ float4 red[4][2][32];
  __shared__ unsigned s_old;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int b = blockIdx.x, t = b >> 2, q = b & 3;
  const int cg = tid & 31, rg = tid >> 5;  // column quad; rows 4 rg .. 4 rg + 3 of the quarter
  const float4* blk = src + (size_t)b * 1024;
  float4 x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = blk[(4 * rg + i) * 32 + cg];
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f), c = a;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * q + 4 * rg + i;
    const float y = own_weight(t, r), z = qs_weight(t, r);
    a.x = fmaf(y, x[i].x, a.x); a.y = fmaf(y, x[i].y, a.y); a.z = fmaf(y, x[i].z, a.z); a.w = fmaf(y, x[i].w, a.w);
    c.x = fmaf(z, x[i].x, c.x); c.y = fmaf(z, x[i].y, c.y); c.z = fmaf(z, x[i].z, c.z); c.w = fmaf(z, x[i].w, c.w);
  }
  a.x += __shfl_xor(a.x, 32); a.y += __shfl_xor(a.y, 32); a.z += __shfl_xor(a.z, 32); a.w += __shfl_xor(a.w, 32);
  c.x += __shfl_xor(c.x, 32); c.y += __shfl_xor(c.y, 32); c.z += __shfl_xor(c.z, 32); c.w += __shfl_xor(c.w, 32);
  if (lane < 32) {
    red[wave][0][lane] = a;
    red[wave][1][lane] = c;
  }
  __syncthreads();
  if (tid < 64) {  // thread (v, quad): v 0 the own_weight sums, 1 the qs_weight sums
    const int v = tid >> 5, qd = tid & 31;
    float4 sum = red[0][v][qd];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float4 o = red[w][v][qd];
      sum.x += o.x; sum.y += o.y; sum.z += o.z; sum.w += o.w;
    }
    reinterpret_cast<float4*>(part + (size_t)b * 256)[tid] = sum;
  }
  if constexpr (EXCHANGE) {
    __threadfence();
    __syncthreads();
    if (tid == 0) s_old = atomicAdd(&cnt[t], 1u);
    __syncthreads();
    if (s_old != 3) return;
    __threadfence();
    if (tid < 64) {
      float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const float4 o = reinterpret_cast<const float4*>(part + ((size_t)t * 4 + qq) * 256)[tid];
        sum.x += o.x; sum.y += o.y; sum.z += o.z; sum.w += o.w;
      }
      reinterpret_cast<float4*>(out + (size_t)t * 256)[tid] = sum;
    }
    if (tid == 0) cnt[t] = 0;  // ready for the next launch on the stream
  }
}

}  // namespace

extern "C" {

// Read `tiles` consecutive tiles of `tile_bytes` each (16384, 32768 or 65536)
// starting at `src` (device, 16-byte aligned), one workgroup per tile.  `sink` is a
// device buffer of at least 1 KiB, written only in the impossible case above.
// Returns 0, -1 for bad arguments, -4 if the launch failed.
int dl_probe_tile_read(const void* src, int tile_bytes, int tiles, void* sink, void* stream) {
  if (!src || !sink || tiles <= 0 || !aligned16(src)) return -1;
  return launch<0>(const_cast<void*>(src), nullptr, 0, 0, tile_bytes, tiles, sink, static_cast<hipStream_t>(stream));
}

// As dl_probe_tile_read, and each workgroup also reads the first `log_bytes` bytes
// (a multiple of 16, at most 65536) of its tile's region of `log`, whose regions are
// `log_stride` bytes apart (a multiple of 16, >= log_bytes).
int dl_probe_tile_read_log(const void* src, int tile_bytes, int tiles, const void* log, int log_bytes,
                           int log_stride, void* sink, void* stream) {
  if (!src || !log || !sink || tiles <= 0 || !aligned16(src) || !aligned16(log)) return -1;
  if (log_bytes < 0 || log_bytes % 16 || log_bytes > 16 * kThreads * kMaxLogPieces || log_stride % 16 ||
      log_stride < log_bytes)
    return -1;
  return launch<1>(const_cast<void*>(src), log, log_bytes / 16, log_stride / 16, tile_bytes, tiles, sink,
                   static_cast<hipStream_t>(stream));
}

// Read `units` consecutive 16 KiB units at `src` (device, 16-byte aligned) with
// `wgs` persistent workgroups of 256 threads (64 KiB of LDS each), three units in
// flight per workgroup.  Returns 0, -1 for bad arguments, -4 if the launch failed.
int dl_probe_tile_stream(const void* src, int units, int wgs, void* sink, void* stream) {
  if (!src || !sink || units <= 0 || wgs <= 0 || !aligned16(src)) return -1;
  tile_stream_kernel<<<wgs, kStreamThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const float4*>(src), units, static_cast<float*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Stream `tiles` 128 x 128 fp32 tiles at `src` (device, 16-byte aligned, 64 KiB each)
// through LDS with `wgs` persistent workgroups of 320 threads (130 KiB of LDS each, so
// one per CU) and write their column sums, as defined at owned_stream_kernel, to `out`
// (device, tiles x 128 floats).  order 0: whole tiles per workgroup, strided; 1: the
// pool's 16 KiB units strided over the workgroups (needs tiles % wgs == 0); 2: as 0, each
// tile's units in a rotated order; 3: contiguous runs of whole tiles per workgroup.
// Returns 0, -1 for bad arguments, -4 if the launch failed.
int dl_probe_owned_stream(const void* src, int tiles, int order, void* out, int wgs, void* stream) {
  if (!src || !out || tiles <= 0 || wgs <= 0 || !aligned16(src) || !aligned16(out)) return -1;
  if (order < 0 || order > 3) return -1;
  if (order == 1 && tiles % wgs) return -1;
  auto st = static_cast<hipStream_t>(stream);
  const float4* s = static_cast<const float4*>(src);
  float* o = static_cast<float*>(out);
  if (order == 0) owned_stream_kernel<0><<<wgs, kOwnThreads, 0, st>>>(s, tiles, o);
  else if (order == 1) owned_stream_kernel<1><<<wgs, kOwnThreads, 0, st>>>(s, tiles, o);
  else if (order == 2) owned_stream_kernel<2><<<wgs, kOwnThreads, 0, st>>>(s, tiles, o);
  else owned_stream_kernel<3><<<wgs, kOwnThreads, 0, st>>>(s, tiles, o);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Quarter-split column sums of `tiles` 128 x 128 fp32 tiles at `src` (device, 16-byte
// aligned), one 256-thread workgroup per 16 KiB quarter, as defined at
// quarter_split_kernel: the partials go to `part` (device, tiles x 4 x 256 floats); with
// `exchange` nonzero the four partials of each tile are also added up inside the launch
// into `out` (device, tiles x 256 floats), counted in `cnt` (device, tiles unsigned
// ints, all zero on entry; left zero).  Returns 0, -1 for bad arguments, -4 if the launch
// failed.
int dl_probe_quarter_split(const void* src, int tiles, int exchange, void* part, void* cnt, void* out,
                           void* stream) {
  if (!src || !part || tiles <= 0 || !aligned16(src) || !aligned16(part)) return -1;
  if (exchange && (!cnt || !out || !aligned16(out))) return -1;
  if (static_cast<int64_t>(tiles) * 4 > INT32_MAX) return -1;
  auto st = static_cast<hipStream_t>(stream);
  const float4* s = static_cast<const float4*>(src);
  if (exchange)
    quarter_split_kernel<true><<<tiles * 4, 256, 0, st>>>(s, static_cast<float*>(part), static_cast<unsigned*>(cnt),
                                                          static_cast<float*>(out));
  else
    quarter_split_kernel<false><<<tiles * 4, 256, 0, st>>>(s, static_cast<float*>(part), nullptr, nullptr);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Read each tile and write it back in place (scaled by 1 - 2^-24, rounded).
int dl_probe_tile_rw(void* src, int tile_bytes, int tiles, void* stream) {
  if (!src || tiles <= 0 || !aligned16(src)) return -1;
  return launch<2>(src, nullptr, 0, 0, tile_bytes, tiles, nullptr, static_cast<hipStream_t>(stream));
}

}  // extern "C"
