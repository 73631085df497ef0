// Read-rate probe for the benchmark (libdlprobe.so, not part of the decode library).
//
// One workgroup of 256 threads per tile reads the tile's bytes once (16-byte
// loads, all issued before any is used) and keeps nothing: the access shape of
// the decode step's base read with nothing else around it.  Timing it over the
// very pools the decode step reads gives the rate the memory system delivers
// for that shape, launch size and cache state, measured in the same run as the
// decode step.  The loaded values feed a sum that is stored only if it equals a
// value no sum of finite inputs hits in practice, so the loads cannot be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

template <int FPT>
__global__ void __launch_bounds__(256) tile_read_kernel(const float4* __restrict__ src, float* sink) {
  const size_t base = (size_t)blockIdx.x * 256 * FPT;
  float4 v[FPT];
#pragma unroll
  for (int i = 0; i < FPT; ++i) v[i] = src[base + (size_t)i * 256 + threadIdx.x];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < FPT; ++i) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  if (s == 1.2345678e30f) sink[blockIdx.x & 255] = s;
}

}  // namespace

extern "C" {

// Read `tiles` consecutive tiles of `tile_bytes` each (4096, 16384, 32768 or 65536)
// starting at `src` (device, 16-byte aligned), one workgroup per tile.  `sink` is a
// device buffer of at least 1 KiB that is written only in the impossible case above.
// Returns 0, -1 for bad arguments, -4 if the launch failed.
int dl_probe_tile_read(const void* src, int tile_bytes, int tiles, void* sink, void* stream) {
  if (src == nullptr || sink == nullptr || tiles <= 0 || (reinterpret_cast<uintptr_t>(src) & 15) != 0) return -1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const float4* s = static_cast<const float4*>(src);
  float* k = static_cast<float*>(sink);
  switch (tile_bytes) {
    case 4096: tile_read_kernel<1><<<tiles, 256, 0, st>>>(s, k); break;
    case 16384: tile_read_kernel<4><<<tiles, 256, 0, st>>>(s, k); break;
    case 32768: tile_read_kernel<8><<<tiles, 256, 0, st>>>(s, k); break;
    case 65536: tile_read_kernel<16><<<tiles, 256, 0, st>>>(s, k); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
