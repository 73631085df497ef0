// Matrix-core fold for dl_merge (gfx950).
//
// The same rank-n update as the vector fold in decode.hip ("DeltaLog: Deferred
// Materialization of Recurrent States for Linear Attention Decoding", Abstract:
// periodic merges fold the log of compact updates back into the dense base):
//   B <- diag(2^c_now) B + sum_{e<n} diag(2^(c_now - c_e)) k_e u_e^T
// with c_now the cumulative log2-decay of the newest entry.  Here the whole tile
// stays in registers for the fold, so it is read and written once at any log
// length, and the sum is a product W^T U (W[e][i] = 2^(c_now[i] - c_e[i]) k_e[i],
// U[e][j] = u_e[j]) on v_mfma_f32_16x16x4_f32: fp32 operands, fp32 accumulation,
// four log entries per instruction.
//
// Register layout.  The instruction is issued with the factor block first
// (A[m][k] = U[e0 + k][col m]) and the weights second (B[k][n] = W[e0 + k][row n]),
// so its 16 x 16 result holds, in lane (g, r16) = (lane / 16, lane % 16), rows
// r16 and columns 4g .. 4g + 3 of a 16 x 16 block of the tile: one float4 of one
// state row per lane and block, the layout of a plain 16-byte load of the tile.
#include <type_traits>

#include "dl_device.hpp"
#include "launch.hpp"

namespace dl {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int DK, int DV, bool BF>
struct MfmaFoldGeo {
  // Eight waves on a 64 KiB fp32 tile (eight 16 x 16 blocks a wave), four on the smaller
  // tiles, which measured faster with four (64 x 64: 1.51x against 1.58x the vector unit).
  static constexpr int NT = DK * DV >= 16384 ? 512 : 256;
  static constexpr int NW = NT / 64;
  static constexpr int RB = DK / 16, CB = DV / 16;  // 16 x 16 blocks of the tile
  static constexpr int NWR = RB < NW ? RB : NW;     // waves along the rows
  static constexpr int NWC = NW / NWR;              // and along the columns
  static constexpr int RBW = RB / NWR;              // row blocks per wave
  static constexpr int CBW = CB / NWC;              // column blocks per wave
  // With a bf16 base, column blocks go in pairs so that a lane's eight values of one row
  // (four in each block) are adjacent in memory: one 16-byte load.
  static constexpr bool PAIR = BF;
  static constexpr int ME = 16;  // log entries staged at a time (four instructions deep)
  // LDS row strides of 16 mod 64 words: the four lane groups of one operand read
  // (entries e0 + g, 16 rows or columns each) hit 64 distinct banks.
  static constexpr int WS = DK + 16;
  static constexpr int US = DV + 16;
  static_assert(NWR * RBW == RB && NWC * CBW == CB && (!PAIR || CBW % 2 == 0), "tile geometry");
  // Column of the tile held by index m (0..15) of column block cb: 16 cb + m, or with
  // pairs, 32 (cb / 2) + 8 (m / 4) + 4 (cb % 2) + m % 4.
  __device__ static constexpr int col(int cb, int m) {
    return PAIR ? 32 * (cb / 2) + 8 * (m / 4) + 4 * (cb % 2) + m % 4 : 16 * cb + m;
  }
  // Where the factors of columns c .. c + 3 (c a multiple of 4) go in a staged LDS row:
  // position 16 cb + m holds column col(cb, m), so one operand read is 16 consecutive words.
  __device__ static constexpr int upos(int c) {
    return PAIR ? 16 * (2 * (c / 32) + (c % 8) / 4) + 4 * ((c % 32) / 8) : c;
  }
};

template <int VAR, int DK, int DV, bool BF>
__global__ void __launch_bounds__((MfmaFoldGeo<DK, DV, BF>::NT)) merge_mfma_kernel(PoolArgs p, int min_fill) {
  using G = MfmaFoldGeo<DK, DV, BF>;
  using BIO = BaseIO<BF>;
  constexpr bool VEC = VAR != DL_GDN;  // a decay per key channel
  constexpr int CW = VEC ? DK : 1;     // floats per log_c entry
  using UT = std::conditional_t<VAR == DL_RWKV6, uint16_t, float>;
  using URaw = std::conditional_t<VAR == DL_RWKV6, uint2, float4>;  // four factors, raw
  __shared__ __attribute__((aligned(16))) float s_c[CW];  // c_now, natural order
  __shared__ __attribute__((aligned(16))) float s_g[CW];  // 2^c_now
  __shared__ __attribute__((aligned(16))) float s_w[G::ME * G::WS];
  __shared__ __attribute__((aligned(16))) float s_u[G::ME * G::US];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int wr = wave % G::NWR, wc = wave / G::NWR;  // this wave's row and column block groups
  const int tile = blockIdx.x;
  const int n = p.fill[tile];
  if (n < min_fill || n == 0) return;  // uniform: the whole workgroup leaves
  const size_t lbase = (size_t)tile * p.L;
  const UT* log_u = static_cast<const UT*>(p.log_u);

  // The tile: lane (g, r16) holds row 16 (wr RBW + rb) + r16 and, of column block
  // cb = wc CBW + j, the columns col(cb, 4 g) .. col(cb, 4 g) + 3.
  auto* tb = BIO::tile(p.base, (size_t)tile * DK * DV);
  auto row = [&](int rb) { return 16 * (wr * G::RBW + rb) + r16; };
  f32x4 acc[G::RBW][G::CBW];
#pragma unroll
  for (int rb = 0; rb < G::RBW; ++rb) {
    if constexpr (G::PAIR) {
#pragma unroll
      for (int j = 0; j < G::CBW; j += 2) {
        const uint4 w = *reinterpret_cast<const uint4*>(tb + (size_t)row(rb) * DV + G::col(wc * G::CBW + j, 4 * g));
        const float4 a = widen4(make_uint2(w.x, w.y)), b = widen4(make_uint2(w.z, w.w));
        acc[rb][j] = f32x4{a.x, a.y, a.z, a.w};
        acc[rb][j + 1] = f32x4{b.x, b.y, b.z, b.w};
      }
    } else {
#pragma unroll
      for (int j = 0; j < G::CBW; ++j) {
        const float4 x = BIO::load(tb, ((size_t)row(rb) * DV + G::col(wc * G::CBW + j, 4 * g)) / 4);
        acc[rb][j] = f32x4{x.x, x.y, x.z, x.w};
      }
    }
  }

  for (int i = tid; i < CW; i += G::NT) {
    const float c = p.log_c[(lbase + n - 1) * CW + i];
    s_c[i] = c;
    s_g[i] = exp2f(c);
  }
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < G::RBW; ++rb) {
    const float sc = s_g[VEC ? row(rb) : 0];
#pragma unroll
    for (int j = 0; j < G::CBW; ++j) acc[rb][j] *= sc;
  }

  for (int e0 = 0; e0 < n; e0 += G::ME) {
    const int cnt = min(G::ME, n - e0);
    __syncthreads();  // the previous stage's operand reads are done
    // fold weights, eight channels of one entry per job (zeros past the fill)
    for (int job = tid; job < G::ME * DK / 8; job += G::NT) {
      const int m = job / (DK / 8), i0 = (job % (DK / 8)) * 8, e = e0 + m;
      float w[8];
      if (m < cnt) {
        float kf[8];
        unpack8(*reinterpret_cast<const uint4*>(p.log_k + (lbase + e) * DK + i0), kf);
        if constexpr (VEC) {
          float ce[8];
          load8(p.log_c + (lbase + e) * DK + i0, ce);
#pragma unroll
          for (int i = 0; i < 8; ++i) w[i] = exp2f(s_c[i0 + i] - ce[i]) * kf[i];
        } else {
          const float sc = exp2f(s_c[0] - p.log_c[lbase + e]);
#pragma unroll
          for (int i = 0; i < 8; ++i) w[i] = sc * kf[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = 0.f;
      }
      float4* dst = reinterpret_cast<float4*>(s_w + m * G::WS + i0);
      dst[0] = make_float4(w[0], w[1], w[2], w[3]);
      dst[1] = make_float4(w[4], w[5], w[6], w[7]);
    }
    // update factors, four columns of one entry per job
    for (int job = tid; job < G::ME * DV / 4; job += G::NT) {
      const int m = job / (DV / 4), j0 = (job % (DV / 4)) * 4;
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
      if (m < cnt) u = widen4(*reinterpret_cast<const URaw*>(log_u + (lbase + e0 + m) * DV + j0));
      *reinterpret_cast<float4*>(s_u + m * G::US + G::upos(j0)) = u;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < G::ME / 4; ++ks) {
      if (4 * ks >= cnt) break;  // uniform
      const int m = 4 * ks + g;  // this lane group's entry
      float bw[G::RBW];
#pragma unroll
      for (int rb = 0; rb < G::RBW; ++rb) bw[rb] = s_w[m * G::WS + row(rb)];
#pragma unroll
      for (int j = 0; j < G::CBW; ++j) {
        const float au = s_u[m * G::US + 16 * (wc * G::CBW + j) + r16];
#pragma unroll
        for (int rb = 0; rb < G::RBW; ++rb)
          acc[rb][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(au, bw[rb], acc[rb][j], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int rb = 0; rb < G::RBW; ++rb) {
    if constexpr (G::PAIR) {
#pragma unroll
      for (int j = 0; j < G::CBW; j += 2) {
        const f32x4 a = acc[rb][j], b = acc[rb][j + 1];
        const uint4 w = make_uint4(f32_to_bf16_rne(a[0]) | (f32_to_bf16_rne(a[1]) << 16),
                                   f32_to_bf16_rne(a[2]) | (f32_to_bf16_rne(a[3]) << 16),
                                   f32_to_bf16_rne(b[0]) | (f32_to_bf16_rne(b[1]) << 16),
                                   f32_to_bf16_rne(b[2]) | (f32_to_bf16_rne(b[3]) << 16));
        *reinterpret_cast<uint4*>(tb + (size_t)row(rb) * DV + G::col(wc * G::CBW + j, 4 * g)) = w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < G::CBW; ++j) {
        const f32x4 x = acc[rb][j];
        BIO::store(tb, ((size_t)row(rb) * DV + G::col(wc * G::CBW + j, 4 * g)) / 4,
                   make_float4(x[0], x[1], x[2], x[3]));
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
