// Eager decode step for gfx950: read the whole state, update it, write it back.
//
// This is the comparator the DeltaLog page ("DeltaLog: Deferred
// Materialization of Recurrent States for Linear Attention Decoding",
// Abstract) measures against: the usual decoder rewrites the whole recurrent
// state in memory after each token it generates.  Per (sequence, head)
// tile, with d the decay (alpha for GDN, a dk-vector for KDA and RWKV6):
//   GDN/KDA  p = (diag(d) S)^T k,  u = beta (v - p),  S' = diag(d) S + k u^T,
//            o = S'^T q = (diag(d) S)^T q + (k . q) u
//   RWKV6    o = S^T r + (sum_i r_i bonus_i k_i) v,  S' = diag(w) S + k v^T
// One read and one write of the 64 KiB tile (at dk = dv = 128); the tile stays
// in registers between the reduction and the write.
#include "dl_device.hpp"
#include "launch.hpp"

namespace dl {

template <int VAR, int DK, int DV>
__global__ void __launch_bounds__((Geo<DK, DV>::NT)) eager_kernel(float* state, StepArgs s, int heads) {
  using G = Geo<DK, DV>;
  constexpr bool VEC = VAR != DL_GDN;
  constexpr int RPT = G::RPT;
  const int tid = threadIdx.x;
  const int tile = blockIdx.x;

  __shared__ __attribute__((aligned(16))) float s_d[DK];   // decay per key row
  __shared__ __attribute__((aligned(16))) float s_k[DK];   // k
  __shared__ __attribute__((aligned(16))) float s_yk[DK];  // d . k   (RWKV6: unused)
  __shared__ __attribute__((aligned(16))) float s_yq[DK];  // d . q   (RWKV6: r)
  __shared__ float s_dot;
  __shared__ float s_kk;  // ||k||^2 (Kaczmarz step size)
  __shared__ float s_red[G::NW][2][DV];
  __shared__ __attribute__((aligned(16))) float s_u[DV];

  // small loads by the first LPE lanes: 8 channels each
  const int ch = tid % G::LPE;
  const size_t in_off = (size_t)tile * DK + ch * 8;
  const uint4 kt8 = *reinterpret_cast<const uint4*>(s.k + in_off);
  const uint4 qt8 = *reinterpret_cast<const uint4*>(s.q + in_off);
  float dec[8], bonus[8];
  if constexpr (VEC) {
    const float4* dp = reinterpret_cast<const float4*>(s.decay + in_off);
    const float4 d0 = dp[0], d1 = dp[1];
    dec[0] = d0.x; dec[1] = d0.y; dec[2] = d0.z; dec[3] = d0.w;
    dec[4] = d1.x; dec[5] = d1.y; dec[6] = d1.z; dec[7] = d1.w;
  } else {
    const float a = s.decay[tile];
#pragma unroll
    for (int i = 0; i < 8; ++i) dec[i] = a;
  }
  if constexpr (VAR == DL_RWKV6) {
    const float4* bp = reinterpret_cast<const float4*>(s.bonus + (size_t)(tile % heads) * DK + ch * 8);
    const float4 b0 = bp[0], b1 = bp[1];
    bonus[0] = b0.x; bonus[1] = b0.y; bonus[2] = b0.z; bonus[3] = b0.w;
    bonus[4] = b1.x; bonus[5] = b1.y; bonus[6] = b1.z; bonus[7] = b1.w;
  }
  float vcol = 0.f;
  if (tid < DV) vcol = bf16_to_f32(s.v[(size_t)tile * DV + tid]);
  float beta = 0.f;  // the given step size, or eta for the Kaczmarz one
  if constexpr (VAR != DL_RWKV6) beta = s.eta ? s.eta[tile] : s.beta[tile];

  const int rg = tid / G::CG, cg = tid % G::CG;
  float4 B[RPT];
  float4* bp = reinterpret_cast<float4*>(state + ((size_t)tile * DK + rg * RPT) * DV) + cg;
#pragma unroll
  for (int r = 0; r < RPT; ++r) B[r] = bp[(size_t)r * (DV / 4)];

  if (tid < G::LPE) {
    float kt[8], qt[8];
    unpack8(kt8, kt);
    unpack8(qt8, qt);
    float d = 0.f, kk = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      s_d[ch * 8 + i] = dec[i];
      s_k[ch * 8 + i] = kt[i];
      if constexpr (VAR == DL_RWKV6) {
        s_yq[ch * 8 + i] = qt[i];
        d = fmaf(qt[i] * bonus[i], kt[i], d);
      } else {
        s_yk[ch * 8 + i] = dec[i] * kt[i];
        s_yq[ch * 8 + i] = dec[i] * qt[i];
        d = fmaf(kt[i], qt[i], d);
        kk = fmaf(kt[i], kt[i], kk);
      }
    }
    d = group_sum<G::LPE>(d);
    kk = group_sum<G::LPE>(kk);
    if (tid == 0) {
      s_dot = d;
      s_kk = kk;
    }
  }
  __syncthreads();

  float4 ak = make_float4(0.f, 0.f, 0.f, 0.f), aq = ak;
  {
    const float* yk = s_yk + rg * RPT;
    const float* yq = s_yq + rg * RPT;
#pragma unroll
    for (int r = 0; r < RPT; r += 4) {
      const float4 q4 = *reinterpret_cast<const float4*>(yq + r);
      aq = f4_fma(q4.x, B[r + 0], aq);
      aq = f4_fma(q4.y, B[r + 1], aq);
      aq = f4_fma(q4.z, B[r + 2], aq);
      aq = f4_fma(q4.w, B[r + 3], aq);
      if constexpr (VAR != DL_RWKV6) {
        const float4 k4 = *reinterpret_cast<const float4*>(yk + r);
        ak = f4_fma(k4.x, B[r + 0], ak);
        ak = f4_fma(k4.y, B[r + 1], ak);
        ak = f4_fma(k4.z, B[r + 2], ak);
        ak = f4_fma(k4.w, B[r + 3], ak);
      }
    }
  }
  aq.x = colgroup_sum<G::CG>(aq.x);
  aq.y = colgroup_sum<G::CG>(aq.y);
  aq.z = colgroup_sum<G::CG>(aq.z);
  aq.w = colgroup_sum<G::CG>(aq.w);
  if constexpr (VAR != DL_RWKV6) {
    ak.x = colgroup_sum<G::CG>(ak.x);
    ak.y = colgroup_sum<G::CG>(ak.y);
    ak.z = colgroup_sum<G::CG>(ak.z);
    ak.w = colgroup_sum<G::CG>(ak.w);
  }
  const int wave = tid / 64, lane = tid % 64;
  if (lane < G::CG) {
    *reinterpret_cast<float4*>(&s_red[wave][1][cg * 4]) = aq;
    if constexpr (VAR != DL_RWKV6) *reinterpret_cast<float4*>(&s_red[wave][0][cg * 4]) = ak;
  }
  __syncthreads();
  if (tid < DV) {
    float pk = 0.f, oq = 0.f;
#pragma unroll
    for (int w = 0; w < G::NW; ++w) {
      oq += s_red[w][1][tid];
      if constexpr (VAR != DL_RWKV6) pk += s_red[w][0][tid];
    }
    float u, o;
    if constexpr (VAR == DL_RWKV6) {
      u = vcol;
      o = fmaf(s_dot, vcol, oq);
    } else {
      // Kaczmarz step size (Kaczmarz Linear Attention abstract): beta = eta / (||k||^2 + eps)
      const float b = s.eta ? beta / (s_kk + s.eps) : beta;
      u = b * (vcol - pk);
      o = fmaf(s_dot, u, oq);
    }
    s.out[(size_t)tile * DV + tid] = o;
    s_u[tid] = u;
  }
  __syncthreads();
  const float4 u4 = *reinterpret_cast<const float4*>(s_u + cg * 4);
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int row = rg * RPT + r;
    const float d = s_d[row], kr = s_k[row];
    bp[(size_t)r * (DV / 4)] = f4_fma(kr, u4, f4_mul(B[r], d));
  }
}

hipError_t launch_eager(int variant, int dk, int dv, int tiles, int heads, float* state, const StepArgs& s,
                        hipStream_t stream) {
  hipError_t err = hipSuccess;
  float* st = state;
  StepArgs sa = s;
  int h = heads;
  void* args[] = {&st, &sa, &h};
#define CALL_EAGER(V, K, D)                                                                    \
  err = hipLaunchKernel(reinterpret_cast<const void*>(&eager_kernel<V, K, D>), dim3(tiles),    \
                        dim3(Geo<K, D>::NT), args, 0, stream)
  if (variant == DL_GDN) {
    if (dk == 128 && dv == 128) CALL_EAGER(DL_GDN, 128, 128);
    else if (dk == 64 && dv == 64) CALL_EAGER(DL_GDN, 64, 64);
    else if (dk == 128) CALL_EAGER(DL_GDN, 128, 64);
    else CALL_EAGER(DL_GDN, 64, 128);
  } else if (variant == DL_KDA) {
    if (dk == 128 && dv == 128) CALL_EAGER(DL_KDA, 128, 128);
    else if (dk == 64 && dv == 64) CALL_EAGER(DL_KDA, 64, 64);
    else if (dk == 128) CALL_EAGER(DL_KDA, 128, 64);
    else CALL_EAGER(DL_KDA, 64, 128);
  } else {
    if (dk == 128 && dv == 128) CALL_EAGER(DL_RWKV6, 128, 128);
    else if (dk == 64 && dv == 64) CALL_EAGER(DL_RWKV6, 64, 64);
    else if (dk == 128) CALL_EAGER(DL_RWKV6, 128, 64);
    else CALL_EAGER(DL_RWKV6, 64, 128);
  }
#undef CALL_EAGER
  return err;
}

}  // namespace dl
