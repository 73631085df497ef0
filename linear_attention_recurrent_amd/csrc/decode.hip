// DeltaLog decode step, merge and pool initialisation kernels for gfx950.
//
// The recurrences and the deferred form are those declared in deltalog.h:
// a dense base B plus a bounded log of rank-1 updates (k_j, u_j, c_j), with
// c the cumulative log2-decay since the last merge ("DeltaLog: Deferred
// Materialization of Recurrent States for Linear Attention Decoding",
// Abstract: dense base state plus a bounded log of recent compact updates,
// appends on most steps, periodic merges into the base).
//
// Decode step, per (sequence, head) tile, n = entries in the log:
//   reads   r_k = B^T (2^c_t . k_t)  and  r_q = B^T (2^c_t . q_t)   one pass over B
//           sigma^k_j = sum_i k_j[i] 2^(c_t[i]-c_j[i]) k_t[i]  (and sigma^q_j with q_t)
//   GDN/KDA u_t = beta (v_t - r_k - sum_j sigma^k_j u_j)     the delta-rule residual write
//           o_t = r_q + sum_j sigma^q_j u_j + (k_t . q_t) u_t  output of the updated state
//   RWKV6   o_t = B^T(2^c_{t-1} . r_t) + sum_j sigma^r_j v_j + (sum_i r_i bonus_i k_i) v_t
//           (sigma^r_j with c_{t-1}: the readout sees the state before the write)
//   append  (k_t, u_t, c_t) to slot n, unless n + 1 == L: then fold all L
//           updates into B (B <- diag(2^c_t) B + sum_j diag(2^(c_t-c_j)) k_j u_j^T)
//           and reset the fill to 0.
// The base is read once and written only by folding steps; a non-folding step
// writes the output, one log entry and the fill.
#include <type_traits>

#include "dl_device.hpp"
#include "launch.hpp"

namespace dl {

// Fold log entries [0, nlog) of a tile, plus the current step's update when
// has_cur, into the base rows held in registers.  s_cnow is the cumulative
// log2-decay to fold at (LDS, 1 or DK floats), s_kcur / s_ucur the current
// update's key and factor (LDS).  s_w / s_uu are LDS staging areas of MC*DK and
// MC*DV floats.  Must be called by every thread of the workgroup.
template <int VAR, int DK, int DV, int RPT>
__device__ __forceinline__ void fold_into(float4 (&B)[RPT], const PoolArgs& p, int tile,
                                          int nlog, const float* s_cnow, bool has_cur,
                                          const float* s_kcur, const float* s_ucur, float* s_w,
                                          float* s_uu) {
  using G = Geo<DK, DV>;
  static_assert(RPT == G::RPT, "register tile");
  const int tid = threadIdx.x;
  const int rg = tid / G::CG, cg = tid % G::CG;
  const size_t lbase = (size_t)tile * p.L;

  if constexpr (VAR == DL_GDN) {
    const float g = exp2f(s_cnow[0]);
#pragma unroll
    for (int r = 0; r < RPT; ++r) B[r] = f4_mul(B[r], g);
  } else {
#pragma unroll
    for (int r = 0; r < RPT; ++r) B[r] = f4_mul(B[r], exp2f(s_cnow[rg * RPT + r]));
  }

  const int total = nlog + (has_cur ? 1 : 0);
  for (int m0 = 0; m0 < total; m0 += G::MC) {
    for (int idx = tid; idx < G::MC * DK; idx += G::NT) {
      const int m = idx / DK, i = idx % DK, e = m0 + m;
      float w = 0.f;
      if (e < nlog) {
        const float kj = bf16_to_f32(p.log_k[(lbase + e) * DK + i]);
        const float dc = (VAR == DL_GDN) ? (s_cnow[0] - p.log_c[lbase + e])
                                         : (s_cnow[i] - p.log_c[(lbase + e) * DK + i]);
        w = exp2f(dc) * kj;
      } else if (e == nlog && has_cur) {
        w = s_kcur[i];
      }
      s_w[m * DK + i] = w;
    }
    for (int idx = tid; idx < G::MC * DV; idx += G::NT) {
      const int m = idx / DV, j = idx % DV, e = m0 + m;
      float u = 0.f;
      if (e < nlog) {
        if constexpr (VAR == DL_RWKV6)
          u = bf16_to_f32(static_cast<const uint16_t*>(p.log_u)[(lbase + e) * DV + j]);
        else
          u = static_cast<const float*>(p.log_u)[(lbase + e) * DV + j];
      } else if (e == nlog && has_cur) {
        u = s_ucur[j];
      }
      s_uu[m * DV + j] = u;
    }
    __syncthreads();
    const int mcount = min(G::MC, total - m0);
    for (int m = 0; m < mcount; ++m) {
      const float4 u4 = *reinterpret_cast<const float4*>(s_uu + m * DV + cg * 4);
      const float* wr = s_w + m * DK + rg * RPT;
#pragma unroll
      for (int r = 0; r < RPT; r += 4) {
        const float4 w4 = *reinterpret_cast<const float4*>(wr + r);
        B[r + 0] = f4_fma(w4.x, u4, B[r + 0]);
        B[r + 1] = f4_fma(w4.y, u4, B[r + 1]);
        B[r + 2] = f4_fma(w4.z, u4, B[r + 2]);
        B[r + 3] = f4_fma(w4.w, u4, B[r + 3]);
      }
    }
    __syncthreads();
  }
}

// Read coefficients of one log entry j, computed by a group of LPE lanes that
// each hold 8 key channels:
//   GDN    sigma^k_j = 2^(c_t - c_j) (k_j . k_t),   sigma^q_j = 2^(c_t - c_j) (k_j . q_t)
//   KDA    sigma^k_j = sum_i k_j[i] 2^(c_t[i] - c_j[i]) k_t[i]   (sigma^q_j with q_t)
//   RWKV6  sigma^r_j = sum_i k_j[i] 2^(c_{t-1}[i] - c_j[i]) r_t[i]
// Lane 0 of the group stores them to s_sig[0][j] and s_sig[1][j].
template <int VAR, int LPE, int CWN>
__device__ __forceinline__ void log_coefs(const uint4 kj8, const float (&cj)[CWN], const float (&kt)[8],
                                          const float (&qt)[8], const float (&ct)[CWN],
                                          const float (&cprev)[CWN], float (*s_sig)[DL_MAX_LOG_LEN],
                                          int j, int ch) {
  float kj[8];
  unpack8(kj8, kj);
  float a = 0.f, b = 0.f;
  if constexpr (VAR == DL_GDN) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a = fmaf(kj[i], kt[i], a);
      b = fmaf(kj[i], qt[i], b);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = kj[i] * exp2f((VAR == DL_RWKV6 ? cprev[i] : ct[i]) - cj[i]);
      a = fmaf(e, VAR == DL_RWKV6 ? qt[i] : kt[i], a);
      if constexpr (VAR == DL_KDA) b = fmaf(e, qt[i], b);
    }
  }
  a = group_sum<LPE>(a);
  if constexpr (VAR != DL_RWKV6) b = group_sum<LPE>(b);
  if (ch == 0) {
    if constexpr (VAR == DL_GDN) {
      const float sc = exp2f(ct[0] - cj[0]);
      s_sig[0][j] = sc * a;
      s_sig[1][j] = sc * b;
    } else {
      s_sig[0][j] = a;
      s_sig[1][j] = b;
    }
  }
}

template <int VAR, int DK, int DV>
__global__ void __launch_bounds__((Geo<DK, DV>::NT)) decode_kernel(PoolArgs p, StepArgs s) {
  using G = Geo<DK, DV>;
  constexpr bool VEC = VAR != DL_GDN;  // per-key-channel decay
  constexpr int CW = VEC ? DK : 1;     // floats per log_c entry
  constexpr int RPT = G::RPT;
  using UT = std::conditional_t<VAR == DL_RWKV6, uint16_t, float>;

  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  const int L = p.L;
  const int n = p.fill[tile];  // same for the whole workgroup
  const bool due = (n + 1 == L);
  const size_t lbase = (size_t)tile * L;
  const UT* log_u = static_cast<const UT*>(p.log_u);

  __shared__ float s_kt[DK];                   // k_t
  __shared__ float s_yk[DK];                   // 2^c_t . k_t   (RWKV6: 2^c_{t-1} . r_t)
  __shared__ float s_yq[DK];                   // 2^c_t . q_t   (GDN/KDA)
  __shared__ float s_ct[CW];                   // c_t
  __shared__ float s_sig[2][DL_MAX_LOG_LEN];   // sigma^k_j, sigma^q_j (RWKV6: sigma^r_j)
  __shared__ float s_dot;                      // k_t . q_t  (RWKV6: sum r bonus k)
  __shared__ float s_red[G::NW][2][DV];        // per-wave column partial sums
  __shared__ float s_u[DV];                    // u_t (RWKV6: v_t)
  __shared__ __attribute__((aligned(16))) float s_w[G::MC * DK];
  __shared__ __attribute__((aligned(16))) float s_uu[G::MC * DV];

  // ---- 1. small loads first: they are consumed while the base is in flight.
  // All of them are unconditional (slot indices are clamped into [0, L), which
  // init_state zeroed), so no branch forces a wait before the base loads issue;
  // entries beyond the fill are masked out where they are used.
  // "Entry lanes": group eg of LPE lanes works on log entry eg (+NG, ...), lane ch on
  // channels [8ch, 8ch+8).
  const int eg = tid / G::LPE, ch = tid % G::LPE;
  const size_t in_off = (size_t)tile * DK + ch * 8;
  const uint4 kt8 = *reinterpret_cast<const uint4*>(s.k + in_off);
  const uint4 qt8 = *reinterpret_cast<const uint4*>(s.q + in_off);
  const int prev = n > 0 ? n - 1 : 0;     // slot of the newest entry (read only if n > 0)
  const int e0 = eg < L ? eg : L - 1;     // first-pass entry slot of this lane group
  float dec[VEC ? 8 : 1], cprev[VEC ? 8 : 1], cj[VEC ? 8 : 1];
  float bonus[VAR == DL_RWKV6 ? 8 : 1];
  if constexpr (VEC) {
    load8(s.decay + in_off, dec);
    load8(p.log_c + (lbase + prev) * DK + ch * 8, cprev);
    load8(p.log_c + (lbase + e0) * DK + ch * 8, cj);
  } else {
    dec[0] = s.decay[tile];
    cprev[0] = p.log_c[lbase + prev];
    cj[0] = p.log_c[lbase + e0];
  }
  if constexpr (VAR == DL_RWKV6) load8(s.bonus + (size_t)(tile % p.heads) * DK + ch * 8, bonus);
  const uint4 kj8 = *reinterpret_cast<const uint4*>(p.log_k + (lbase + e0) * DK + ch * 8);
  // "Tile lanes": thread (rg, cg) owns rows [rg*RPT, +RPT) x columns [4cg, 4cg+4).
  const int rg = tid / G::CG, cg = tid % G::CG;
  using URaw = std::conditional_t<VAR == DL_RWKV6, uint2, float4>;  // 4 factors, raw
  URaw up[G::UPF];
#pragma unroll
  for (int e = 0; e < G::UPF; ++e) {
    const int j = min(rg + G::RG * e, L - 1);
    up[e] = *reinterpret_cast<const URaw*>(log_u + (lbase + j) * DV + cg * 4);
  }
  // column lanes: v_t and beta
  const uint16_t vbits = s.v[(size_t)tile * DV + (tid % DV)];
  float beta = 0.f;
  if constexpr (VAR != DL_RWKV6) beta = s.beta[tile];
  uint4 v8 = make_uint4(0, 0, 0, 0);  // RWKV6 appends v_t's bf16 bits
  if constexpr (VAR == DL_RWKV6)
    v8 = *reinterpret_cast<const uint4*>(s.v + (size_t)tile * DV + (tid % (DV / 8)) * 8);

  // ---- 2. the base tile: RPT float4 loads per thread, all in flight at once.
  float4 B[RPT];
  {
    const float4* bp = reinterpret_cast<const float4*>(p.base + ((size_t)tile * DK + rg * RPT) * DV) + cg;
#pragma unroll
    for (int r = 0; r < RPT; ++r) B[r] = bp[(size_t)r * (DV / 4)];
  }

  // ---- 3. decay bookkeeping, scaled read vectors and log coefficients (entry lanes).
  float kt[8], qt[8];
  unpack8(kt8, kt);
  unpack8(qt8, qt);
  float ct[VEC ? 8 : 1];
  float gsc[8];  // 2^c_t per channel (RWKV6: 2^c_{t-1})
#pragma unroll
  for (int i = 0; i < (VEC ? 8 : 1); ++i) cprev[i] = n > 0 ? cprev[i] : 0.f;
  if constexpr (VEC) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ct[i] = cprev[i] + step_log2_decay(dec[i]);
      gsc[i] = exp2f(VAR == DL_RWKV6 ? cprev[i] : ct[i]);
    }
  } else {
    ct[0] = cprev[0] + step_log2_decay(dec[0]);
    const float g = exp2f(ct[0]);
#pragma unroll
    for (int i = 0; i < 8; ++i) gsc[i] = g;
  }
  if (eg == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      s_kt[ch * 8 + i] = kt[i];
      s_yk[ch * 8 + i] = gsc[i] * (VAR == DL_RWKV6 ? qt[i] : kt[i]);
      if constexpr (VAR != DL_RWKV6) s_yq[ch * 8 + i] = gsc[i] * qt[i];
      if constexpr (VEC) s_ct[ch * 8 + i] = ct[i];
    }
    if constexpr (!VEC) {
      if (ch == 0) s_ct[0] = ct[0];
    }
  }
  {
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (VAR == DL_RWKV6) d = fmaf(qt[i] * bonus[i], kt[i], d);
      else d = fmaf(kt[i], qt[i], d);
    }
    d = group_sum<G::LPE>(d);
    if (tid == 0) s_dot = d;
  }
  // first pass: entry eg, from the registers loaded above
  if (eg < n) log_coefs<VAR, G::LPE>(kj8, cj, kt, qt, ct, cprev, s_sig, eg, ch);
  // later passes, only when L > NG + 1
  for (int j = eg + G::NG; j < n; j += G::NG) {
    float cjj[VEC ? 8 : 1];
    if constexpr (VEC) load8(p.log_c + (lbase + j) * DK + ch * 8, cjj);
    else cjj[0] = p.log_c[lbase + j];
    const uint4 kjj = *reinterpret_cast<const uint4*>(p.log_k + (lbase + j) * DK + ch * 8);
    log_coefs<VAR, G::LPE>(kjj, cjj, kt, qt, ct, cprev, s_sig, j, ch);
  }
  __syncthreads();

  // ---- 4. column sums: log part, then the base matvec (tile lanes).
  float4 ak = make_float4(0.f, 0.f, 0.f, 0.f), aq = ak;
#pragma unroll
  for (int e = 0; e < G::UPF; ++e) {
    const int j = rg + G::RG * e;
    if (j < n) {
      const float4 uj = widen4(up[e]);
      ak = f4_fma(s_sig[0][j], uj, ak);
      if constexpr (VAR != DL_RWKV6) aq = f4_fma(s_sig[1][j], uj, aq);
    }
  }
  for (int j = rg + G::RG * G::UPF; j < n; j += G::RG) {  // only when L > RG*UPF + 1
    const float4 uj = widen4(*reinterpret_cast<const URaw*>(log_u + (lbase + j) * DV + cg * 4));
    ak = f4_fma(s_sig[0][j], uj, ak);
    if constexpr (VAR != DL_RWKV6) aq = f4_fma(s_sig[1][j], uj, aq);
  }
  {
    const float* yk = s_yk + rg * RPT;
    const float* yq = s_yq + rg * RPT;
#pragma unroll
    for (int r = 0; r < RPT; r += 4) {
      const float4 k4 = *reinterpret_cast<const float4*>(yk + r);
      ak = f4_fma(k4.x, B[r + 0], ak);
      ak = f4_fma(k4.y, B[r + 1], ak);
      ak = f4_fma(k4.z, B[r + 2], ak);
      ak = f4_fma(k4.w, B[r + 3], ak);
      if constexpr (VAR != DL_RWKV6) {
        const float4 q4 = *reinterpret_cast<const float4*>(yq + r);
        aq = f4_fma(q4.x, B[r + 0], aq);
        aq = f4_fma(q4.y, B[r + 1], aq);
        aq = f4_fma(q4.z, B[r + 2], aq);
        aq = f4_fma(q4.w, B[r + 3], aq);
      }
    }
  }
  // reduce over the row groups of this wave, then across waves through LDS
  ak.x = colgroup_sum<G::CG>(ak.x);
  ak.y = colgroup_sum<G::CG>(ak.y);
  ak.z = colgroup_sum<G::CG>(ak.z);
  ak.w = colgroup_sum<G::CG>(ak.w);
  if constexpr (VAR != DL_RWKV6) {
    aq.x = colgroup_sum<G::CG>(aq.x);
    aq.y = colgroup_sum<G::CG>(aq.y);
    aq.z = colgroup_sum<G::CG>(aq.z);
    aq.w = colgroup_sum<G::CG>(aq.w);
  }
  const int wave = tid / 64, lane = tid % 64;
  if (lane < G::CG) {
    *reinterpret_cast<float4*>(&s_red[wave][0][cg * 4]) = ak;
    if constexpr (VAR != DL_RWKV6) *reinterpret_cast<float4*>(&s_red[wave][1][cg * 4]) = aq;
  }
  __syncthreads();

  // ---- 5. per-column results, output, append (column lanes / entry lanes).
  if (tid < DV) {
    const float vcol = bf16_to_f32(vbits);
    float pk = 0.f, oq = 0.f;
#pragma unroll
    for (int w = 0; w < G::NW; ++w) {
      pk += s_red[w][0][tid];
      if constexpr (VAR != DL_RWKV6) oq += s_red[w][1][tid];
    }
    float o, u;
    if constexpr (VAR == DL_RWKV6) {
      u = vcol;
      o = fmaf(s_dot, vcol, pk);
    } else {
      u = beta * (vcol - pk);
      o = fmaf(s_dot, u, oq);
      if (!due) static_cast<float*>(p.log_u)[(lbase + n) * DV + tid] = u;
    }
    s.out[(size_t)tile * DV + tid] = o;
    s_u[tid] = u;
  }
  if (!due) {
    if (eg == 0) {
      *reinterpret_cast<uint4*>(p.log_k + (lbase + n) * DK + ch * 8) = kt8;
      if constexpr (VEC) {
        float4* cp = reinterpret_cast<float4*>(p.log_c + (lbase + n) * DK + ch * 8);
        cp[0] = make_float4(ct[0], ct[1], ct[2], ct[3]);
        cp[1] = make_float4(ct[4], ct[5], ct[6], ct[7]);
      } else {
        if (ch == 0) p.log_c[lbase + n] = ct[0];
      }
    }
    if constexpr (VAR == DL_RWKV6) {
      if (tid < DV / 8)
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.log_u) + (lbase + n) * DV + tid * 8) = v8;
    }
    if (tid == 0) p.fill[tile] = n + 1;
    return;
  }

  // ---- 6. folding step: B <- diag(2^c_t) B + sum_j diag(2^(c_t-c_j)) k_j u_j^T + k_t u_t^T.
  __syncthreads();
  fold_into<VAR, DK, DV, RPT>(B, p, tile, n, s_ct, true, s_kt, s_u, s_w, s_uu);
  {
    float4* bp = reinterpret_cast<float4*>(p.base + ((size_t)tile * DK + rg * RPT) * DV) + cg;
#pragma unroll
    for (int r = 0; r < RPT; ++r) bp[(size_t)r * (DV / 4)] = B[r];
  }
  if (tid == 0) p.fill[tile] = 0;
}

// dl_merge: fold the logs of tiles holding at least min_fill entries.
template <int VAR, int DK, int DV>
__global__ void __launch_bounds__((Geo<DK, DV>::NT)) merge_kernel(PoolArgs p, int min_fill) {
  using G = Geo<DK, DV>;
  constexpr bool VEC = VAR != DL_GDN;
  constexpr int CW = VEC ? DK : 1;
  constexpr int RPT = G::RPT;
  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  const int n = p.fill[tile];
  if (n < min_fill || n == 0) return;  // uniform: the whole workgroup leaves
  const size_t lbase = (size_t)tile * p.L;

  __shared__ float s_c[CW];
  __shared__ __attribute__((aligned(16))) float s_w[G::MC * DK];
  __shared__ __attribute__((aligned(16))) float s_uu[G::MC * DV];

  const int rg = tid / G::CG, cg = tid % G::CG;
  float4 B[RPT];
  const float4* bp = reinterpret_cast<const float4*>(p.base + ((size_t)tile * DK + rg * RPT) * DV) + cg;
#pragma unroll
  for (int r = 0; r < RPT; ++r) B[r] = bp[(size_t)r * (DV / 4)];
  for (int i = tid; i < CW; i += G::NT) s_c[i] = p.log_c[(lbase + n - 1) * CW + i];
  __syncthreads();
  fold_into<VAR, DK, DV, RPT>(B, p, tile, n, s_c, false, nullptr, nullptr, s_w, s_uu);
  float4* wp = reinterpret_cast<float4*>(p.base + ((size_t)tile * DK + rg * RPT) * DV) + cg;
#pragma unroll
  for (int r = 0; r < RPT; ++r) wp[(size_t)r * (DV / 4)] = B[r];
  if (tid == 0) p.fill[tile] = 0;
}

// dl_init_state: copy or zero the base and zero every log slot of each tile.
template <int VAR, int DK, int DV>
__global__ void __launch_bounds__(256) init_kernel(PoolArgs p, const float* init_base) {
  constexpr int CW = (VAR == DL_GDN) ? 1 : DK;
  constexpr int USZ = (VAR == DL_RWKV6) ? 2 : 4;
  const int tid = threadIdx.x;
  const size_t tile = blockIdx.x;
  const size_t L = p.L;
  float4* dst = reinterpret_cast<float4*>(p.base + tile * DK * DV);
  const float4* src = init_base ? reinterpret_cast<const float4*>(init_base + tile * DK * DV) : nullptr;
  if (src != dst) {
    for (int i = tid; i < DK * DV / 4; i += 256)
      dst[i] = src ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const uint4 z = make_uint4(0, 0, 0, 0);
  uint4* lk = reinterpret_cast<uint4*>(p.log_k + tile * L * DK);
  for (size_t i = tid; i < L * DK * 2 / 16; i += 256) lk[i] = z;
  uint4* lu = reinterpret_cast<uint4*>(static_cast<char*>(p.log_u) + tile * L * DV * USZ);
  for (size_t i = tid; i < L * DV * USZ / 16; i += 256) lu[i] = z;
  float* lc = p.log_c + tile * L * CW;
  for (size_t i = tid; i < L * CW; i += 256) lc[i] = 0.f;
}

// ------------------------------------------------------------------ launchers
#define DL_DISPATCH(VAR_, DK_, DV_, CALL)                                  \
  do {                                                                     \
    if ((DK_) == 128 && (DV_) == 128) { CALL(VAR_, 128, 128); }            \
    else if ((DK_) == 64 && (DV_) == 64) { CALL(VAR_, 64, 64); }           \
    else if ((DK_) == 128 && (DV_) == 64) { CALL(VAR_, 128, 64); }         \
    else { CALL(VAR_, 64, 128); }                                          \
  } while (0)

#define DL_VARIANTS(VARI, DK_, DV_, CALL)                                  \
  do {                                                                     \
    if ((VARI) == DL_GDN) DL_DISPATCH(DL_GDN, DK_, DV_, CALL);             \
    else if ((VARI) == DL_KDA) DL_DISPATCH(DL_KDA, DK_, DV_, CALL);        \
    else DL_DISPATCH(DL_RWKV6, DK_, DV_, CALL);                            \
  } while (0)

hipError_t launch_decode(int variant, int dk, int dv, int tiles, const PoolArgs& p, const StepArgs& s,
                         hipStream_t stream) {
  hipError_t err = hipSuccess;
  PoolArgs pa = p;
  StepArgs sa = s;
  void* args[] = {&pa, &sa};
#define CALL_DECODE(V, K, D)                                                                    \
  err = hipLaunchKernel(reinterpret_cast<const void*>(&decode_kernel<V, K, D>), dim3(tiles),    \
                        dim3(Geo<K, D>::NT), args, 0, stream)
  DL_VARIANTS(variant, dk, dv, CALL_DECODE);
#undef CALL_DECODE
  return err;
}

hipError_t launch_merge(int variant, int dk, int dv, int tiles, const PoolArgs& p, int min_fill,
                        hipStream_t stream) {
  hipError_t err = hipSuccess;
  PoolArgs pa = p;
  int mf = min_fill;
  void* args[] = {&pa, &mf};
#define CALL_MERGE(V, K, D)                                                                    \
  err = hipLaunchKernel(reinterpret_cast<const void*>(&merge_kernel<V, K, D>), dim3(tiles),    \
                        dim3(Geo<K, D>::NT), args, 0, stream)
  DL_VARIANTS(variant, dk, dv, CALL_MERGE);
#undef CALL_MERGE
  return err;
}

hipError_t launch_init(int variant, int dk, int dv, int tiles, const PoolArgs& p, const float* init_base,
                       hipStream_t stream) {
  hipError_t err = hipSuccess;
  PoolArgs pa = p;
  const float* ib = init_base;
  void* args[] = {&pa, &ib};
#define CALL_INIT(V, K, D)                                                                     \
  err = hipLaunchKernel(reinterpret_cast<const void*>(&init_kernel<V, K, D>), dim3(tiles),     \
                        dim3(256), args, 0, stream)
  DL_VARIANTS(variant, dk, dv, CALL_INIT);
#undef CALL_INIT
  return err;
}

}  // namespace dl
