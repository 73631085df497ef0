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

// Read each tile and write it back in place (scaled by 1 - 2^-24, rounded).
int dl_probe_tile_rw(void* src, int tile_bytes, int tiles, void* stream) {
  if (!src || tiles <= 0 || !aligned16(src)) return -1;
  return launch<2>(src, nullptr, 0, 0, tile_bytes, tiles, nullptr, static_cast<hipStream_t>(stream));
}

}  // extern "C"
