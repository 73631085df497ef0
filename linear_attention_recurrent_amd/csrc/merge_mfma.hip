// Matrix-core fold for dl_merge (gfx950).
//
// The same rank-n update as the vector fold in decode.hip ("DeltaLog: Deferred
// Materialization of Recurrent States for Linear Attention Decoding", Abstract:
// a merge folds the logged low-rank updates into the base from time to time):
//   B <- diag(2^c_now) B + sum_{e<n} diag(2^(c_now - c_e)) k_e u_e^T
// with c_now the cumulative log2-decay of the newest entry.  Here the whole tile
// stays in registers for the fold, so it is read and written once at any log
// length, and each entry's rank-1 term goes through v_mfma_f32_4x4x1_16b_f32
// (sixteen independent 4 x 4 x 1 products per instruction, fp32 operands and
// accumulation): one instruction adds u_e[cols] w_e[rows] to 16 blocks of 4 rows x
// 4 columns, w_e[i] = 2^(c_now[i] - c_e[i]) k_e[i].
//
// Register layout.  Block b (lanes 4b .. 4b + 3) takes the factors as its first
// operand (lane 4b + m supplies the factor of column m of the block) and the weights
// as its second (lane 4b + r supplies the weight of row r), so lane 4b + r holds row r
// and the block's four columns: one float4 of one state row, the layout of a 16-byte
// load.  The 16 blocks of an instruction cover the same four rows and 64 consecutive
// columns, so a wave's load or store instruction moves four rows x 256 bytes of the
// tile (the 16 x 16 x 4 instruction would give 16 rows x 64 bytes).
#include <type_traits>

#include "dl_device.hpp"
#include "launch.hpp"

namespace dl {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int DK, int DV, bool BF>
struct MfmaFoldGeo {
  static constexpr int NW = DK / 16;  // waves: each owns 16 consecutive rows
  static constexpr int NT = NW * 64;
  static constexpr int RQ = 4;        // four-row groups per wave
  static constexpr int NCG = DV / 64; // 64-column groups
  // With a bf16 base and dv = 128, the two column groups interleave by fours so that a
  // lane's eight values of one row are adjacent in memory: one 16-byte load.
  static constexpr bool PAIR = BF && NCG == 2;
  static constexpr int ME = 16;       // log entries staged at a time
  static constexpr int WS = DK + 4;   // LDS row strides (words)
  static constexpr int US = DV + 4;
  // Column held by index m (0..3) of block b (0..15) in column group c.
  __device__ static constexpr int col(int c, int b, int m) { return PAIR ? 8 * b + 4 * c + m : 64 * c + 4 * b + m; }
  // Where the factors of columns j .. j + 3 (j a multiple of 4) go in a staged LDS row:
  // position 64 c + 4 b + m holds column col(c, b, m), so one operand read is 64 consecutive words.
  __device__ static constexpr int upos(int j) { return PAIR ? 64 * ((j / 4) % 2) + 4 * (j / 8) : j; }
};

template <int VAR, int DK, int DV, bool BF>
__global__ void __launch_bounds__((MfmaFoldGeo<DK, DV, BF>::NT)) merge_mfma_kernel(PoolArgs p, int min_fill) {
  using G = MfmaFoldGeo<DK, DV, BF>;
  using BIO = BaseIO<BF>;
  constexpr bool VEC = VAR != DL_GDN;  // a decay per key channel
  constexpr int CW = VEC ? DK : 1;     // floats per log_c entry
  using UT = std::conditional_t<VAR == DL_RWKV6, uint16_t, float>;
  using URaw = std::conditional_t<VAR == DL_RWKV6, uint2, float4>;  // four factors, raw
  __shared__ __attribute__((aligned(16))) float s_g[CW];  // 2^c_now
  __shared__ __attribute__((aligned(16))) float s_w[G::ME * G::WS];
  __shared__ __attribute__((aligned(16))) float s_u[G::ME * G::US];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = lane >> 2, r4 = lane & 3;  // block and row within the four-row group
  const int tile = blockIdx.x;
  const int n = p.fill[tile];
  if (n < min_fill || n <= 0 || n >= p.L) return;  // uniform: the whole workgroup leaves
  const size_t lbase = (size_t)tile * p.L;
  const UT* log_u = static_cast<const UT*>(p.log_u);

  // Stage entries [e0, e0 + cnt) into LDS: fold weights (eight channels of one entry per
  // job, c_now read from the newest entry directly) and factors (four columns per job).
  const float* cnow = p.log_c + (lbase + n - 1) * CW;
  auto stage = [&](int e0, int cnt) {
    for (int job = tid; job < cnt * DK / 8; job += G::NT) {
      const int m = job / (DK / 8), i0 = (job % (DK / 8)) * 8, e = e0 + m;
      float w[8];
      float kf[8];
      unpack8(*reinterpret_cast<const uint4*>(p.log_k + (lbase + e) * DK + i0), kf);
      if constexpr (VEC) {
        float ce[8], cn[8];
        load8(p.log_c + (lbase + e) * DK + i0, ce);
        load8(cnow + i0, cn);
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = exp2f(cn[i] - ce[i]) * kf[i];
      } else {
        const float sc = exp2f(cnow[0] - p.log_c[lbase + e]);
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = sc * kf[i];
      }
      float4* dst = reinterpret_cast<float4*>(s_w + m * G::WS + i0);
      dst[0] = make_float4(w[0], w[1], w[2], w[3]);
      dst[1] = make_float4(w[4], w[5], w[6], w[7]);
    }
    for (int job = tid; job < cnt * DV / 4; job += G::NT) {
      const int m = job / (DV / 4), j0 = (job % (DV / 4)) * 4;
      const float4 u = widen4(*reinterpret_cast<const URaw*>(log_u + (lbase + e0 + m) * DV + j0));
      *reinterpret_cast<float4*>(s_u + m * G::US + G::upos(j0)) = u;
    }
  };
  auto fold = [&](int cnt, f32x4 (&acc)[G::RQ][G::NCG]) {
    for (int m = 0; m < cnt; ++m) {  // one entry per instruction
      float bw[G::RQ], au[G::NCG];
#pragma unroll
      for (int q = 0; q < G::RQ; ++q) bw[q] = s_w[m * G::WS + 16 * wave + 4 * q + r4];
#pragma unroll
      for (int c = 0; c < G::NCG; ++c) au[c] = s_u[m * G::US + 64 * c + lane];
#pragma unroll
      for (int q = 0; q < G::RQ; ++q)
#pragma unroll
        for (int c = 0; c < G::NCG; ++c)
          acc[q][c] = __builtin_amdgcn_mfma_f32_4x4x1f32(au[c], bw[q], acc[q][c], 0, 0, 0);
    }
  };

  // The small loads first: the first stage's log inputs are issued ahead of the tile and
  // waited for alone, so their LDS stores are made while the tile streams in.  Slots past
  // the stage read zeros through out-of-range buffer offsets (no branch around a load).
  const int cnt0 = min(G::ME, n);
  constexpr int JW = (G::ME * DK / 8 + G::NT - 1) / G::NT;  // weight jobs per thread
  constexpr int JU = (G::ME * DV / 4 + G::NT - 1) / G::NT;  // factor jobs per thread
  const auto rk = make_rsrc(p.log_k + lbase * DK, (uint32_t)(p.L * DK * 2));
  const auto rc = make_rsrc(p.log_c + lbase * CW, (uint32_t)(p.L * CW * 4));
  const auto ru = make_rsrc(log_u + lbase * DV, (uint32_t)(p.L * DV * sizeof(UT)));
  uint4 k8[JW];
  float ce[JW][VEC ? 8 : 1], cn[JW][VEC ? 8 : 1];
  float4 u4[JU];
#pragma unroll
  for (int jw = 0; jw < JW; ++jw) {
    const int job = tid + jw * G::NT, m = job / (DK / 8), i0 = (job % (DK / 8)) * 8;
    const bool ok = m < cnt0;
    k8[jw] = bload16(rk, ok ? (uint32_t)((m * DK + i0) * 2) : kOutOfRange);
    if constexpr (VEC) {
      bload8f(rc, ok ? (uint32_t)((m * DK + i0) * 4) : kOutOfRange, ce[jw]);
      bload8f(rc, (uint32_t)(((n - 1) * DK + i0) * 4), cn[jw]);
    } else {
      ce[jw][0] = bload4f(rc, ok ? (uint32_t)(m * 4) : kOutOfRange);
      cn[jw][0] = bload4f(rc, (uint32_t)((n - 1) * 4));
    }
  }
#pragma unroll
  for (int ju = 0; ju < JU; ++ju) {
    const int job = tid + ju * G::NT, m = job / (DV / 4), j0 = (job % (DV / 4)) * 4;
    u4[ju] = bload_factor4(ru, m < cnt0 ? (uint32_t)((m * DV + j0) * sizeof(UT)) : kOutOfRange, UT{});
  }
  __builtin_amdgcn_sched_barrier(0);

  // The tile: lane (b, r4) holds row 16 wave + 4 q + r4, columns col(c, b, 0..3).
  auto* tb = BIO::tile(p.base, (size_t)tile * DK * DV);
  auto row = [&](int q) { return 16 * wave + 4 * q + r4; };
  f32x4 acc[G::RQ][G::NCG];
#pragma unroll
  for (int q = 0; q < G::RQ; ++q) {
    if constexpr (G::PAIR) {
      const uint4 w = *reinterpret_cast<const uint4*>(tb + (size_t)row(q) * DV + G::col(0, b, 0));
      const float4 x = widen4(make_uint2(w.x, w.y)), y = widen4(make_uint2(w.z, w.w));
      acc[q][0] = f32x4{x.x, x.y, x.z, x.w};
      acc[q][1] = f32x4{y.x, y.y, y.z, y.w};
    } else {
#pragma unroll
      for (int c = 0; c < G::NCG; ++c) {
        const float4 x = BIO::load(tb, ((size_t)row(q) * DV + G::col(c, b, 0)) / 4);
        acc[q][c] = f32x4{x.x, x.y, x.z, x.w};
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // the first stage into LDS, and the scale
#pragma unroll
  for (int jw = 0; jw < JW; ++jw) {
    const int job = tid + jw * G::NT, m = job / (DK / 8), i0 = (job % (DK / 8)) * 8;
    if (m < cnt0) {
      float kf[8], w[8];
      unpack8(k8[jw], kf);
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = exp2f(cn[jw][VEC ? i : 0] - ce[jw][VEC ? i : 0]) * kf[i];
      float4* dst = reinterpret_cast<float4*>(s_w + m * G::WS + i0);
      dst[0] = make_float4(w[0], w[1], w[2], w[3]);
      dst[1] = make_float4(w[4], w[5], w[6], w[7]);
    }
  }
#pragma unroll
  for (int ju = 0; ju < JU; ++ju) {
    const int job = tid + ju * G::NT, m = job / (DV / 4), j0 = (job % (DV / 4)) * 4;
    if (m < cnt0) *reinterpret_cast<float4*>(s_u + m * G::US + G::upos(j0)) = u4[ju];
  }
  for (int i = tid; i < CW; i += G::NT) s_g[i] = exp2f(cnow[i]);
  __syncthreads();
#pragma unroll
  for (int q = 0; q < G::RQ; ++q) {
    const float sc = s_g[VEC ? row(q) : 0];
#pragma unroll
    for (int c = 0; c < G::NCG; ++c) acc[q][c] *= sc;
  }
  fold(cnt0, acc);
  for (int e0 = G::ME; e0 < n; e0 += G::ME) {
    const int cnt = min(G::ME, n - e0);
    __syncthreads();  // the previous stage's operand reads are done
    stage(e0, cnt);
    __syncthreads();
    fold(cnt, acc);
  }

#pragma unroll
  for (int q = 0; q < G::RQ; ++q) {
    if constexpr (G::PAIR) {
      const f32x4 x = acc[q][0], y = acc[q][1];
      const uint4 w = make_uint4(f32_to_bf16_rne(x[0]) | (f32_to_bf16_rne(x[1]) << 16),
                                 f32_to_bf16_rne(x[2]) | (f32_to_bf16_rne(x[3]) << 16),
                                 f32_to_bf16_rne(y[0]) | (f32_to_bf16_rne(y[1]) << 16),
                                 f32_to_bf16_rne(y[2]) | (f32_to_bf16_rne(y[3]) << 16));
      *reinterpret_cast<uint4*>(tb + (size_t)row(q) * DV + G::col(0, b, 0)) = w;
    } else {
#pragma unroll
      for (int c = 0; c < G::NCG; ++c) {
        const f32x4 x = acc[q][c];
        BIO::store(tb, ((size_t)row(q) * DV + G::col(c, b, 0)) / 4, make_float4(x[0], x[1], x[2], x[3]));
      }
    }
  }
  if (tid == 0) p.fill[tile] = 0;
}

}  // namespace

hipError_t launch_merge_mfma(int variant, bool bf16_base, int dk, int dv, int tiles, const PoolArgs& p,
                             int min_fill, hipStream_t stream) {
  hipError_t err = hipSuccess;
  PoolArgs pa = p;
  int mf = min_fill;
  void* args[] = {&pa, &mf};
  auto go = [&](const void* fn, int nt) { err = hipLaunchKernel(fn, dim3(tiles), dim3(nt), args, 0, stream); };
#define DL_MF_GO(V, K, D, B) \
  go(reinterpret_cast<const void*>(&merge_mfma_kernel<V, K, D, B>), MfmaFoldGeo<K, D, B>::NT)
#define DL_MF_SHAPES(V, B)                                  \
  do {                                                      \
    if (dk == 128 && dv == 128) DL_MF_GO(V, 128, 128, B);   \
    else if (dk == 64 && dv == 64) DL_MF_GO(V, 64, 64, B);  \
    else if (dk == 128 && dv == 64) DL_MF_GO(V, 128, 64, B); \
    else DL_MF_GO(V, 64, 128, B);                           \
  } while (0)
#define DL_MF_BASES(V)                 \
  do {                                 \
    if (bf16_base) DL_MF_SHAPES(V, true); \
    else DL_MF_SHAPES(V, false);       \
  } while (0)
  if (variant == DL_GDN) DL_MF_BASES(DL_GDN);
  else if (variant == DL_KDA) DL_MF_BASES(DL_KDA);
  else DL_MF_BASES(DL_RWKV6);
#undef DL_MF_BASES
#undef DL_MF_SHAPES
#undef DL_MF_GO
  return err;
}

}  // namespace dl
