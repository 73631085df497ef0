// DeltaLog decode step, merge and pool initialisation kernels for gfx950.
//
// The recurrences and the deferred form are those declared in deltalog.h:
// a dense base B plus a bounded log of rank-1 updates (k_j, u_j, c_j), with
// c the cumulative log2-decay since the last merge ("DeltaLog: Deferred
// Materialization of Recurrent States for Linear Attention Decoding",
// Abstract: the state is a dense base and a length-bounded log of low-rank
// updates; most steps only add to the log, and a merge now and then folds it
// into the base).
//
// Decode step, per (sequence, head) tile, n = entries in the log:
//   reads   r_k = B^T (2^c_t . k_t)  and  r_q = B^T (2^c_t . q_t)   one streamed pass over B
//           sigma^k_j = sum_i k_j[i] 2^(c_t[i]-c_j[i]) k_t[i]  (and sigma^q_j with q_t)
//   GDN/KDA u_t = beta (v_t - r_k - sum_j sigma^k_j u_j)     the delta-rule residual write
//           o_t = r_q + sum_j sigma^q_j u_j + (k_t . q_t) u_t  output of the updated state
//   RWKV6   o_t = B^T(2^c_{t-1} . r_t) + sum_j sigma^r_j v_j + (sum_i r_i bonus_i k_i) v_t
//           (sigma^r_j with c_{t-1}: the readout sees the state before the write)
//   append  (k_t, u_t, c_t) to slot n, unless n + 1 == L: then fold all L
//           updates into B (B <- diag(2^c_t) B + sum_j diag(2^(c_t-c_j)) k_j u_j^T)
//           in a second streamed pass over B, and reset the fill to 0.
// A non-folding step reads the base once and writes only the output, one log
// entry and the fill.
#include <type_traits>

#include "dl_device.hpp"
#include "launch.hpp"

namespace dl {

#ifdef DL_TRACE
// Per-workgroup timestamps, in the opt-in tracing build only (libdeltalog_trace.so):
// s_memrealtime (a 100 MHz clock shared by every CU) at the workgroup's start (0), after
// the barrier that ends the log-coefficient phase (1), after the barrier that ends the
// column sums (2) and at its end (3), plus its hardware id (4), for workgroups < 65,536
// of two launches: the buffer is chosen by the parity of the step's query pointer over
// the slot size tiles * dk * 2 bytes, so consecutive steps of an input pool that holds
// the steps back to back alternate between the two.
__device__ unsigned long long g_trace[2][65536][5];
__device__ __forceinline__ void trace_stamp(int k, const void* q, int tiles, int dk) {
  if (threadIdx.x == 0 && blockIdx.x < 65536) {
    const int par = (int)(((uintptr_t)q / ((size_t)tiles * dk * 2)) & 1);
    g_trace[par][blockIdx.x][k] = __builtin_amdgcn_s_memrealtime();
    if (k == 3) {
      unsigned hw, xcc;
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
      g_trace[par][blockIdx.x][4] = ((unsigned long long)xcc << 32) | hw;
    }
  }
}
#define DL_STAMP(k) trace_stamp(k, s.q, p.tiles, DK)
#else
#define DL_STAMP(k) ((void)0)
#endif

// Threads per workgroup of the decode step (PF: its log prefetch) and of the merge (PF 0)
// at 128 x 128 with an fp32 base, where 512 threads halve each thread's share of the tile:
//   GDN: 512 (80 VGPRs: three workgroups per CU, six waves per SIMD where 256 threads at
//     131 VGPRs give three; cold steps 0.5-1.2 % faster, the vector merge up to 11 %);
//   KDA with PF 0 or 32 (logs of up to 33 entries): 512, held to 128 VGPRs (four waves per
//     SIMD, step_waves) so that two workgroups share a CU: 16 waves where 256 threads at
//     146 VGPRs give 12 (cold steps 3.7 % faster at L = 16, 3.3 % at L = 32); with 64
//     prefetched entries the cap spills.
// Otherwise the geometry's default: with a bf16 base the GDN step was 4 % slower at 512
// threads and the KDA vector merge up to 14 %.
template <int VAR, int DK, int DV, bool BF, int PF>
constexpr int step_threads() {
  return DK * DV < 16384 || BF ? 0 : VAR == DL_GDN || (VAR == DL_KDA && PF <= 32) ? 512 : 0;
}
// Waves per SIMD the register budget must allow: 4 for KDA at 512 threads (above), else
// no bound.
template <int VAR, int DK, int DV, bool BF, int PF>
constexpr int step_waves() {
  return VAR != DL_KDA || DK * DV < 16384 ? 1 : step_threads<VAR, DK, DV, BF, PF>() == 512 ? 4 : 1;
}
template <int VAR, int DK, int DV, bool BF, int PF = 0>
using StepGeo = SGeo<DK, DV, PF, step_threads<VAR, DK, DV, BF, PF>()>;

// Read coefficients of one log entry j, computed by a group of LPE lanes that
// each hold 8 key channels:
//   GDN    sigma^k_j = 2^(c_t - c_j) (k_j . k_t),   sigma^q_j = 2^(c_t - c_j) (k_j . q_t)
//   KDA    sigma^k_j = sum_i k_j[i] 2^(c_t[i] - c_j[i]) k_t[i]   (sigma^q_j with q_t)
//   RWKV6  sigma^r_j = sum_i k_j[i] 2^(c_{t-1}[i] - c_j[i]) r_t[i]
// Lane 0 of the group stores them to s_sig[0][j] and s_sig[1][j].  When
// `stage` is set, the group also stores the entry's fold weights
// w_j[i] = 2^(c_t[i] - c_j[i]) k_j[i] to s_w (rows permuted as for a workgroup of NT
// threads, the calling kernel's).
template <int VAR, int DK, int DV, int NT, int CWN>
__device__ __forceinline__ void log_coefs(const uint4 kj8, const float (&cj)[CWN], const float (&kt)[8],
                                          const float (&qt)[8], const float (&ct)[CWN],
                                          const float (&cprev)[CWN], float (*s_sig)[DL_MAX_LOG_LEN],
                                          int j, int ch, bool stage, float* s_w) {
  using G = SGeo<DK, DV, 0, NT>;
  float kj[8];
  unpack8(kj8, kj);
  float a = 0.f, b = 0.f;
  float e[8];  // 2^(c_t - c_j) per channel (GDN: one value)
  if constexpr (VAR == DL_GDN) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a = fmaf(kj[i], kt[i], a);
      b = fmaf(kj[i], qt[i], b);
    }
    const float sc = exp2f(ct[0] - cj[0]);
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = sc;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      e[i] = exp2f(ct[i] - cj[i]);
      if constexpr (VAR == DL_RWKV6) {
        a = fmaf(kj[i] * exp2f(cprev[i] - cj[i]), qt[i], a);
      } else {
        const float w = kj[i] * e[i];
        a = fmaf(w, kt[i], a);
        b = fmaf(w, qt[i], b);
      }
    }
  }
  if (stage) {
#pragma unroll
    for (int i = 0; i < 8; ++i) s_w[j * DK + G::perm(ch * 8 + i)] = e[i] * kj[i];
  }
  a = group_sum<G::LPE>(a);
  if constexpr (VAR != DL_RWKV6) b = group_sum<G::LPE>(b);
  if (ch == 0) {
    if constexpr (VAR == DL_GDN) {
      s_sig[0][j] = e[0] * a;
      s_sig[1][j] = e[0] * b;
    } else {
      s_sig[0][j] = a;
      s_sig[1][j] = b;
    }
  }
}

// Stage fold entries [e0, e0 + cnt) (cnt <= MC) of a tile into s_w / s_uu for a
// fold at cumulative decay s_cnow (LDS, natural channel order).  Entries below
// nlog come from the log: s_w[m][perm(i)] = 2^(c_now[i] - c_e[i]) k_e[i] and
// s_uu[m][j] = u_e[j]; entry nlog, when asked for, is the current update
// (s_kcur, already permuted, and s_ucur).  Every thread takes part: all of its
// loads (16-byte pieces of key, decay and factor rows; slots outside the stage
// read zeros through out-of-range offsets) are issued before any is used.  NT: the
// threads of the calling kernel's workgroup.
template <int VAR, int DK, int DV, int NT, bool HAS_CUR>
__device__ __forceinline__ void stage_entries(const PoolArgs& p, int tile, int e0, int cnt, int nlog,
                                              const float* s_cnow, const float* s_kcur,
                                              const float* s_ucur, float* s_w, float* s_uu) {
  using G = SGeo<DK, DV, 0, NT>;
  constexpr bool VEC = VAR != DL_GDN;
  constexpr int CW = VEC ? DK : 1;
  using UT = std::conditional_t<VAR == DL_RWKV6, uint16_t, float>;
  constexpr int KJ = DK / 8;                             // 8-channel jobs per entry
  constexpr int UJ = DV / 4;                             // 4-column jobs per entry
  constexpr int JW = (G::MC * KJ + G::NT - 1) / G::NT;  // weight jobs per thread
  constexpr int JU = (G::MC * UJ + G::NT - 1) / G::NT;  // factor jobs per thread
  const int tid = threadIdx.x;
  const size_t lbase = (size_t)tile * p.L;
  const UT* log_u = static_cast<const UT*>(p.log_u);
  const auto rk = make_rsrc(p.log_k + lbase * DK, (uint32_t)(p.L * DK * 2));
  const auto rc = make_rsrc(p.log_c + lbase * CW, (uint32_t)(p.L * CW * 4));
  const auto ru = make_rsrc(log_u + lbase * DV, (uint32_t)(p.L * DV * sizeof(UT)));
  uint4 k8[JW];
  float c8[JW][VEC ? 8 : 1];
  float4 u4[JU];
#pragma unroll
  for (int jw = 0; jw < JW; ++jw) {
    const int job = tid + jw * G::NT, m = job / KJ, i0 = (job % KJ) * 8, e = e0 + m;
    const bool ok = m < cnt && (!HAS_CUR || e < nlog);
    k8[jw] = bload16(rk, ok ? (uint32_t)((e * DK + i0) * 2) : kOutOfRange);
    if constexpr (VEC) bload8f(rc, ok ? (uint32_t)((e * DK + i0) * 4) : kOutOfRange, c8[jw]);
    else c8[jw][0] = bload4f(rc, ok ? (uint32_t)(e * 4) : kOutOfRange);
  }
#pragma unroll
  for (int ju = 0; ju < JU; ++ju) {
    const int job = tid + ju * G::NT, m = job / UJ, j0 = (job % UJ) * 4, e = e0 + m;
    const bool ok = m < cnt && (!HAS_CUR || e < nlog);
    u4[ju] = bload_factor4(ru, ok ? (uint32_t)((e * DV + j0) * sizeof(UT)) : kOutOfRange, UT{});
  }
#pragma unroll
  for (int jw = 0; jw < JW; ++jw) {
    const int job = tid + jw * G::NT, m = job / KJ, i0 = (job % KJ) * 8, e = e0 + m;
    if (m < cnt) {
      if (!HAS_CUR || e < nlog) {
        float kf[8];
        unpack8(k8[jw], kf);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          s_w[m * DK + G::perm(i0 + i)] = exp2f(s_cnow[VEC ? i0 + i : 0] - c8[jw][VEC ? i : 0]) * kf[i];
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) s_w[m * DK + G::perm(i0 + i)] = s_kcur[G::perm(i0 + i)];
      }
    }
  }
#pragma unroll
  for (int ju = 0; ju < JU; ++ju) {
    const int job = tid + ju * G::NT, m = job / UJ, j0 = (job % UJ) * 4, e = e0 + m;
    if (m < cnt) {
      float4* dst = reinterpret_cast<float4*>(s_uu + m * DV + j0);
      if (HAS_CUR && e >= nlog) *dst = *reinterpret_cast<const float4*>(s_ucur + j0);
      else *dst = u4[ju];
    }
  }
}

// One streamed fold pass over a tile's base:
//   B[row][cols] <- g[row] B[row][cols] + sum_{m < nent} s_w[m][perm(row)] s_uu[m][cols]
// with g = 2^c (s_g, rows permuted; one value for GDN) when `scale`, else 1.
template <int VAR, int DK, int DV, bool BF>
__device__ __forceinline__ void fold_pass(typename BaseIO<BF>::T* tb, int nent, bool scale, const float* s_g,
                                          const float* s_w, const float* s_uu) {
  using G = StepGeo<VAR, DK, DV, BF>;
  using BIO = BaseIO<BF>;
  constexpr int RPC = G::RPC;
  const int tid = threadIdx.x;
  const int rg = tid / G::CG, cg = tid % G::CG;
  auto gidx = [&](int c, int rr) { return (size_t)((c * RPC + rr) * G::RG + rg) * (DV / 4) + cg; };
  float4 buf[G::NB][RPC];
#pragma unroll
  for (int c = 0; c < G::NB; ++c)
#pragma unroll
    for (int rr = 0; rr < RPC; ++rr) buf[c][rr] = BIO::load(tb, gidx(c, rr));
#pragma unroll
  for (int c = 0; c < G::NC; ++c) {
    float g[RPC];
    if constexpr (VAR == DL_GDN) {
#pragma unroll
      for (int rr = 0; rr < RPC; ++rr) g[rr] = scale ? s_g[0] : 1.f;
    } else {
      const float4 g4 = scale ? *reinterpret_cast<const float4*>(s_g + rg * G::RPT + c * RPC)
                              : make_float4(1.f, 1.f, 1.f, 1.f);
      g[0] = g4.x; g[1] = g4.y; g[2] = g4.z; g[3] = g4.w;
    }
    float4 x[RPC];
#pragma unroll
    for (int rr = 0; rr < RPC; ++rr) x[rr] = f4_mul(buf[c % G::NB][rr], g[rr]);
    if (c + G::NB < G::NC) {
#pragma unroll
      for (int rr = 0; rr < RPC; ++rr) buf[c % G::NB][rr] = BIO::load(tb, gidx(c + G::NB, rr));
    }
    for (int m = 0; m < nent; ++m) {
      const float4 u4 = *reinterpret_cast<const float4*>(s_uu + m * DV + cg * 4);
      const float4 w4 = *reinterpret_cast<const float4*>(s_w + m * DK + rg * G::RPT + c * RPC);
      x[0] = f4_fma(w4.x, u4, x[0]);
      x[1] = f4_fma(w4.y, u4, x[1]);
      x[2] = f4_fma(w4.z, u4, x[2]);
      x[3] = f4_fma(w4.w, u4, x[3]);
    }
#pragma unroll
    for (int rr = 0; rr < RPC; ++rr) BIO::store(tb, gidx(c, rr), x[rr]);
  }
}

// Fold a tile's nlog logged entries, plus the current update when HAS_CUR,
// into its base, in stages of MC entries loaded from the log (used when the
// fold's entries are not already staged).  Each stage streams the base once;
// a thread re-reads only what it wrote itself in the previous stage.
template <int VAR, int DK, int DV, bool BF, bool HAS_CUR>
__device__ __forceinline__ void fold_staged(const PoolArgs& p, int tile, int nlog,
                                            const float* s_ct, const float* s_g, const float* s_kcur,
                                            const float* s_ucur, float* s_w, float* s_uu) {
  using G = StepGeo<VAR, DK, DV, BF>;
  auto* tb = BaseIO<BF>::tile(p.base, (size_t)tile * DK * DV);
  const int total = nlog + (HAS_CUR ? 1 : 0);
  for (int e0 = 0; e0 < total; e0 += G::MC) {
    const int cnt = min(G::MC, total - e0);
    __syncthreads();  // the previous stage's LDS reads are done
    stage_entries<VAR, DK, DV, G::NT, HAS_CUR>(p, tile, e0, cnt, nlog, s_ct, s_kcur, s_ucur, s_w, s_uu);
    __syncthreads();
    fold_pass<VAR, DK, DV, BF>(tb, cnt, e0 == 0, s_g, s_w, s_uu);
  }
}

// LDS of one decode workgroup.  Per-row vectors are stored with rows permuted
// (SGeo::perm) so that the RPC rows of one chunk of one thread are adjacent.
template <int DK, int DV, int CW, int NW, int MC>
struct DecodeLds {
  __attribute__((aligned(16))) float yk[DK];    // 2^c_t . k_t (RWKV6: 2^c_{t-1} . r_t), permuted
  __attribute__((aligned(16))) float yq[DK];    // 2^c_t . q_t (GDN/KDA), permuted
  __attribute__((aligned(16))) float g[CW];     // 2^c_t, permuted (fold scale)
  __attribute__((aligned(16))) float ct[CW];    // c_t, natural order
  __attribute__((aligned(16))) float kcur[DK];  // k_t, permuted (staged folds)
  __attribute__((aligned(16))) float ucur[DV];  // u_t (staged folds)
  float sig[2][DL_MAX_LOG_LEN];                 // sigma^k_j, sigma^q_j (RWKV6: sigma^r_j)
  float dot;                                    // k_t . q_t  (RWKV6: sum r bonus k)
  float kk;                                     // ||k_t||^2 (Kaczmarz step size)
  __attribute__((aligned(16))) float red[NW][2][DV];  // per-wave column partial sums
  __attribute__((aligned(16))) float w[MC * DK];      // fold weights, permuted rows
  __attribute__((aligned(16))) float uu[MC * DV];     // fold factors
};

// One decode step of one tile.  FOLD is the step whose update fills the log:
// it keeps the whole base tile in registers (one read), folds every update
// into it and writes it back once.  Otherwise the base is streamed in chunks
// and only the output, one log entry and the fill are written.
template <int VAR, int DK, int DV, bool BF, int PF, bool FOLD, typename Lds>
__device__ __forceinline__ void decode_tile(const PoolArgs& p, const StepArgs& s, int tile, int n, Lds& sh) {
  using G = StepGeo<VAR, DK, DV, BF, PF>;
  using BIO = BaseIO<BF>;
  constexpr bool VEC = VAR != DL_GDN;  // per-key-channel decay
  constexpr int CW = VEC ? DK : 1;     // floats per log_c entry
  constexpr int RPC = G::RPC;
  // Base chunks held in registers: the whole tile on a folding step, and for GDN with an
  // fp32 base, whose registers allow it at the same occupancy (the fold already holds the
  // tile), on every step; otherwise NB chunks streamed (a bf16 tile in flight whole was
  // slower).
  constexpr int NBUF = FOLD || (VAR == DL_GDN && !BF) ? G::NC : G::NB;
  using UT = std::conditional_t<VAR == DL_RWKV6, uint16_t, float>;
  using URaw = std::conditional_t<VAR == DL_RWKV6, uint2, float4>;  // 4 log factors, raw

  // Both paths are inlined into one kernel behind a branch on the fill, and the registers
  // it gets are those of the larger: a distinct empty asm with a memory clobber at the head
  // of each keeps the compiler from hoisting their common loads and address arithmetic
  // above the branch, where they were live through the whole of both (RWKV6 64 x 64: 163
  // VGPRs against 116-122 for either path alone, now 133; KDA with a bf16 base 153, now
  // 118, four waves per SIMD instead of three: steps with a bf16 base 1.4 % faster).
  if constexpr (FOLD) asm volatile("; folding step" ::: "memory");
  else asm volatile("; appending step" ::: "memory");
  const int tid = threadIdx.x;
  const int L = p.L;
  const bool reg_stage = FOLD && L <= G::MC;  // the fold's entries come from this pass's registers
  const size_t lbase = (size_t)tile * L;
  const UT* log_u = static_cast<const UT*>(p.log_u);

  // ---- 1. small loads first: they are consumed while the base streams in.
  // Log slots at or past the fill are read through buffer resources with an
  // out-of-range offset: they return zeros without touching memory, and no
  // branch stands between these loads and the base loads below.
  // "Entry lanes": group eg of LPE lanes works on log entry eg (+NG, ...), lane ch
  // on channels [8ch, 8ch+8).
  const int eg = tid / G::LPE, ch = tid % G::LPE;
  const size_t in_off = (size_t)tile * DK + ch * 8;
  const auto rk = make_rsrc(p.log_k + lbase * DK, (uint32_t)(L * DK * 2));
  const auto ru = make_rsrc(log_u + lbase * DV, (uint32_t)(L * DV * sizeof(UT)));
  const auto rc = make_rsrc(p.log_c + lbase * CW, (uint32_t)(L * CW * 4));
  const uint4 kt8 = *reinterpret_cast<const uint4*>(s.k + in_off);
  const uint4 qt8 = *reinterpret_cast<const uint4*>(s.q + in_off);
  // c of the newest entry (zeros when the log is empty)
  const uint32_t prev_off = n > 0 ? (uint32_t)(((n - 1) * CW + (VEC ? ch * 8 : 0)) * 4) : kOutOfRange;
  float dec[VEC ? 8 : 1], cprev[VEC ? 8 : 1];
  float bonus[VAR == DL_RWKV6 ? 8 : 1];
  if constexpr (VEC) {
    load8(s.decay + in_off, dec);
    bload8f(rc, prev_off, cprev);
  } else {
    dec[0] = s.decay[tile];
    cprev[0] = bload4f(rc, prev_off);
  }
  if constexpr (VAR == DL_RWKV6) load8(s.bonus + (size_t)(tile % p.heads) * DK + ch * 8, bonus);
  // the first EPF entry passes of this lane group: entries eg + NG*e (zeros past the fill)
  uint4 kj8[G::EPF];
  float cj[G::EPF][VEC ? 8 : 1];
#pragma unroll
  for (int e = 0; e < G::EPF; ++e) {
    const int j = eg + G::NG * e;
    const bool has = j < n;
    kj8[e] = bload16(rk, has ? (uint32_t)((j * DK + ch * 8) * 2) : kOutOfRange);
    const uint32_t coff = has ? (uint32_t)((j * CW + (VEC ? ch * 8 : 0)) * 4) : kOutOfRange;
    if constexpr (VEC) bload8f(rc, coff, cj[e]);
    else cj[e][0] = bload4f(rc, coff);
  }
  // "Tile lanes": thread (rg, cg) owns columns [4cg, 4cg+4) of rows (c*RPC + rr)*RG + rg.
  const int rg = tid / G::CG, cg = tid % G::CG;
  float4 up[G::UPF];  // factors u_j[4cg..4cg+4) of entries j = rg + RG*e (zeros past the fill)
#pragma unroll
  for (int e = 0; e < G::UPF; ++e) {
    const int j = rg + G::RG * e;
    up[e] = bload_factor4(ru, j < n ? (uint32_t)((j * DV + cg * 4) * sizeof(UT)) : kOutOfRange, UT{});
  }
  const uint16_t vbits = s.v[(size_t)tile * DV + (tid % DV)];  // column lanes: v_t
  float beta = 0.f;  // the given step size, or eta for the Kaczmarz one
  if constexpr (VAR != DL_RWKV6) beta = s.eta ? s.eta[tile] : s.beta[tile];
  uint4 v8 = make_uint4(0, 0, 0, 0);  // RWKV6 appends v_t's bf16 bits
  if constexpr (VAR == DL_RWKV6 && !FOLD)
    v8 = *reinterpret_cast<const uint4*>(s.v + (size_t)tile * DV + (tid % (DV / 8)) * 8);
  // Keep the small loads ahead of the base loads in the issue order: a load that
  // is waited for first must not sit behind the base chunks in the queue.
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. the base: the first NBUF chunks on an appending step.  A folding step
  // loads the whole tile after step 3, so the tile and step 3's registers are
  // not live together.
  auto* tb = BIO::tile(p.base, (size_t)tile * DK * DV);
  auto gidx = [&](int c, int rr) { return (size_t)((c * RPC + rr) * G::RG + rg) * (DV / 4) + cg; };
  float4 buf[NBUF][RPC];
  if constexpr (!FOLD) {
#pragma unroll
    for (int c = 0; c < NBUF; ++c)
#pragma unroll
      for (int rr = 0; rr < RPC; ++rr) buf[c][rr] = BIO::load(tb, gidx(c, rr));
  }

  // ---- 3. decay bookkeeping, scaled read vectors and log coefficients (entry lanes).
  {
    float kt[8], qt[8];
    unpack8(kt8, kt);
    unpack8(qt8, qt);
    float ct[VEC ? 8 : 1];
#pragma unroll
    for (int i = 0; i < (VEC ? 8 : 1); ++i) ct[i] = cprev[i] + step_log2_decay(dec[i]);
    if (eg == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int pi = G::perm(ch * 8 + i);
        const float g = exp2f(ct[VEC ? i : 0]);  // 2^c_t
        if constexpr (VAR == DL_RWKV6) {
          sh.yk[pi] = exp2f(cprev[i]) * qt[i];
        } else {
          sh.yk[pi] = g * kt[i];
          sh.yq[pi] = g * qt[i];
        }
        if constexpr (FOLD) sh.kcur[pi] = kt[i];
        if constexpr (VEC) {
          sh.g[pi] = g;
          sh.ct[ch * 8 + i] = ct[i];
        } else if (ch == 0 && i == 0) {
          sh.g[0] = g;
          sh.ct[0] = ct[0];
        }
        // the current update's fold weight is k_t itself (no decay after it)
        if (reg_stage) sh.w[n * DK + pi] = kt[i];
      }
    }
    float d = 0.f, kk = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (VAR == DL_RWKV6) {
        d = fmaf(qt[i] * bonus[i], kt[i], d);
      } else {
        d = fmaf(kt[i], qt[i], d);
        kk = fmaf(kt[i], kt[i], kk);
      }
    }
    d = group_sum<G::LPE>(d);
    if constexpr (VAR != DL_RWKV6) kk = group_sum<G::LPE>(kk);
    if (tid == 0) {
      sh.dot = d;
      sh.kk = kk;
    }
    // the prefetched passes: entries eg + NG*e, from the registers loaded above
#pragma unroll
    for (int e = 0; e < G::EPF; ++e) {
      const int j = eg + G::NG * e;
      if (j < n) log_coefs<VAR, DK, DV, G::NT>(kj8[e], cj[e], kt, qt, ct, cprev, sh.sig, j, ch, reg_stage, sh.w);
    }
    // later passes, only when L > NG*EPF + 1
    for (int j = eg + G::NG * G::EPF; j < n; j += G::NG) {
      float cjj[VEC ? 8 : 1];
      if constexpr (VEC) load8(p.log_c + (lbase + j) * DK + ch * 8, cjj);
      else cjj[0] = p.log_c[lbase + j];
      const uint4 kjj = *reinterpret_cast<const uint4*>(p.log_k + (lbase + j) * DK + ch * 8);
      log_coefs<VAR, DK, DV, G::NT>(kjj, cjj, kt, qt, ct, cprev, sh.sig, j, ch, false, sh.w);
    }
  }
  if constexpr (FOLD) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < NBUF; ++c)
#pragma unroll
      for (int rr = 0; rr < RPC; ++rr) buf[c][rr] = BIO::load(tb, gidx(c, rr));
  }
  __syncthreads();
  DL_STAMP(1);

  // ---- 4. column sums: the base matvec (streamed, or from the resident tile), then the log part.
  float4 ak = make_float4(0.f, 0.f, 0.f, 0.f), aq = ak;
#pragma unroll
  for (int c = 0; c < G::NC; ++c) {
    float4 x[RPC];
#pragma unroll
    for (int rr = 0; rr < RPC; ++rr) x[rr] = buf[c % NBUF][rr];
    if (!FOLD && c + NBUF < G::NC) {
#pragma unroll
      for (int rr = 0; rr < RPC; ++rr) buf[c % NBUF][rr] = BIO::load(tb, gidx(c + NBUF, rr));
    }
    const float4 k4 = *reinterpret_cast<const float4*>(sh.yk + rg * G::RPT + c * RPC);
    ak = f4_fma(k4.x, x[0], ak);
    ak = f4_fma(k4.y, x[1], ak);
    ak = f4_fma(k4.z, x[2], ak);
    ak = f4_fma(k4.w, x[3], ak);
    if constexpr (VAR != DL_RWKV6) {
      const float4 q4 = *reinterpret_cast<const float4*>(sh.yq + rg * G::RPT + c * RPC);
      aq = f4_fma(q4.x, x[0], aq);
      aq = f4_fma(q4.y, x[1], aq);
      aq = f4_fma(q4.z, x[2], aq);
      aq = f4_fma(q4.w, x[3], aq);
    }
  }
#pragma unroll
  for (int e = 0; e < G::UPF; ++e) {
    const int j = rg + G::RG * e;
    if (j < n) {
      const float4 uj = up[e];
      ak = f4_fma(sh.sig[0][j], uj, ak);
      if constexpr (VAR != DL_RWKV6) aq = f4_fma(sh.sig[1][j], uj, aq);
      if (reg_stage) *reinterpret_cast<float4*>(sh.uu + j * DV + cg * 4) = uj;  // the fold's factors
    }
  }
  for (int j = rg + G::RG * G::UPF; j < n; j += G::RG) {  // only when L > RG*UPF + 1
    const float4 uj = widen4(*reinterpret_cast<const URaw*>(log_u + (lbase + j) * DV + cg * 4));
    ak = f4_fma(sh.sig[0][j], uj, ak);
    if constexpr (VAR != DL_RWKV6) aq = f4_fma(sh.sig[1][j], uj, aq);
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
    *reinterpret_cast<float4*>(&sh.red[wave][0][cg * 4]) = ak;
    if constexpr (VAR != DL_RWKV6) *reinterpret_cast<float4*>(&sh.red[wave][1][cg * 4]) = aq;
  }
  __syncthreads();
  DL_STAMP(2);

  // ---- 5. per-column results, output, append (column lanes / entry lanes).
  if (tid < DV) {
    const float vcol = bf16_to_f32(vbits);
    float pk = 0.f, oq = 0.f;
#pragma unroll
    for (int w = 0; w < G::NW; ++w) {
      pk += sh.red[w][0][tid];
      if constexpr (VAR != DL_RWKV6) oq += sh.red[w][1][tid];
    }
    float o, u;
    if constexpr (VAR == DL_RWKV6) {
      u = vcol;
      o = fmaf(sh.dot, vcol, pk);
    } else {
      // Kaczmarz step size (Kaczmarz Linear Attention abstract): beta = eta / (||k||^2 + eps)
      const float b = s.eta ? beta / (sh.kk + s.eps) : beta;
      u = b * (vcol - pk);
      o = fmaf(sh.dot, u, oq);
      if constexpr (!FOLD) store_res(static_cast<float*>(p.log_u) + lbase * DV, (uint32_t)((n * DV + tid) * 4), u);
    }
    store_res(s.out + (size_t)tile * DV, (uint32_t)(tid * 4), o);
    if constexpr (FOLD) {
      if (reg_stage) sh.uu[n * DV + tid] = u;  // the current update's fold factor
      else sh.ucur[tid] = u;
    }
  }
  if constexpr (!FOLD) {
    if (eg == 0) {
      store_res(p.log_k + lbase * DK, (uint32_t)((n * DK + ch * 8) * 2), kt8);
      if constexpr (VEC) {
        float* cb = p.log_c + lbase * DK;
        store_res(cb, (uint32_t)((n * DK + ch * 8) * 4), *reinterpret_cast<const float4*>(sh.ct + ch * 8));
        store_res(cb, (uint32_t)((n * DK + ch * 8 + 4) * 4), *reinterpret_cast<const float4*>(sh.ct + ch * 8 + 4));
      } else {
        if (ch == 0) store_res(p.log_c + lbase, (uint32_t)(n * 4), sh.ct[0]);
      }
    }
    if constexpr (VAR == DL_RWKV6) {
      if (tid < DV / 8)
        store_res(static_cast<uint16_t*>(p.log_u) + lbase * DV, (uint32_t)((n * DV + tid * 8) * 2), v8);
    }
    if (tid == 0) p.fill[tile] = n + 1;
  } else {
    // ---- 6. folding step, on the resident tile:
    //   B <- diag(2^c_t) B + sum_{j<n} diag(2^(c_t-c_j)) k_j u_j^T + k_t u_t^T
#pragma unroll
    for (int c = 0; c < G::NC; ++c) {
      float g[RPC];
      if constexpr (VEC) {
        const float4 g4 = *reinterpret_cast<const float4*>(sh.g + rg * G::RPT + c * RPC);
        g[0] = g4.x; g[1] = g4.y; g[2] = g4.z; g[3] = g4.w;
      } else {
#pragma unroll
        for (int rr = 0; rr < RPC; ++rr) g[rr] = sh.g[0];
      }
#pragma unroll
      for (int rr = 0; rr < RPC; ++rr) buf[c][rr] = f4_mul(buf[c][rr], g[rr]);
    }
    const int total = n + 1;
    for (int e0 = 0; e0 < total; e0 += G::MC) {
      const int cnt = min(G::MC, total - e0);
      if (!reg_stage) {
        __syncthreads();  // the previous stage's LDS reads are done
        stage_entries<VAR, DK, DV, G::NT, true>(p, tile, e0, cnt, n, sh.ct, sh.kcur, sh.ucur, sh.w, sh.uu);
      }
      __syncthreads();
      for (int m = 0; m < cnt; ++m) {
        const float4 u4 = *reinterpret_cast<const float4*>(sh.uu + m * DV + cg * 4);
#pragma unroll
        for (int c = 0; c < G::NC; ++c) {
          const float4 w4 = *reinterpret_cast<const float4*>(sh.w + m * DK + rg * G::RPT + c * RPC);
          buf[c][0] = f4_fma(w4.x, u4, buf[c][0]);
          buf[c][1] = f4_fma(w4.y, u4, buf[c][1]);
          buf[c][2] = f4_fma(w4.z, u4, buf[c][2]);
          buf[c][3] = f4_fma(w4.w, u4, buf[c][3]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < G::NC; ++c)
#pragma unroll
      for (int rr = 0; rr < RPC; ++rr) BIO::store(tb, gidx(c, rr), buf[c][rr]);
    if (tid == 0) p.fill[tile] = 0;
  }
}

// PF: log entries loaded ahead of the base (the launcher picks it from L so that a
// step finds every entry of its log among them, up to 64).
template <int VAR, int DK, int DV, bool BF, int PF>
__global__ void __launch_bounds__((StepGeo<VAR, DK, DV, BF, PF>::NT), (step_waves<VAR, DK, DV, BF, PF>()))
decode_kernel(PoolArgs p, StepArgs s) {
  using G = StepGeo<VAR, DK, DV, BF, PF>;
  __shared__ DecodeLds<DK, DV, (VAR == DL_GDN ? 1 : DK), G::NW, G::MC> sh;
  DL_STAMP(0);
  const int tile = blockIdx.x;
  const int n = p.fill[tile];  // same for the whole workgroup
  if (n < 0 || n >= p.L) return;  // a fill outside [0, L) (a pool never started): touch nothing
  if (n + 1 == p.L)
    decode_tile<VAR, DK, DV, BF, PF, true>(p, s, tile, n, sh);
  else
    decode_tile<VAR, DK, DV, BF, PF, false>(p, s, tile, n, sh);
#ifdef DL_TRACE
  __syncthreads();
  DL_STAMP(3);
#endif
}

// dl_merge: fold the logs of tiles holding at least min_fill entries.
template <int VAR, int DK, int DV, bool BF>
__global__ void __launch_bounds__((StepGeo<VAR, DK, DV, BF>::NT)) merge_kernel(PoolArgs p, int min_fill) {
  using G = StepGeo<VAR, DK, DV, BF>;
  constexpr bool VEC = VAR != DL_GDN;
  constexpr int CW = VEC ? DK : 1;
  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  const int n = p.fill[tile];
  if (n < min_fill || n <= 0 || n >= p.L) return;  // uniform: the whole workgroup leaves
  const size_t lbase = (size_t)tile * p.L;

  __shared__ __attribute__((aligned(16))) float s_c[CW];  // c of the newest entry, natural order
  __shared__ __attribute__((aligned(16))) float s_g[CW];  // 2^c, permuted
  __shared__ __attribute__((aligned(16))) float s_w[G::MC * DK];
  __shared__ __attribute__((aligned(16))) float s_uu[G::MC * DV];

  for (int i = tid; i < CW; i += G::NT) {
    const float c = p.log_c[(lbase + n - 1) * CW + i];
    s_c[i] = c;
    s_g[VEC ? G::perm(i) : 0] = exp2f(c);
  }
  fold_staged<VAR, DK, DV, BF, false>(p, tile, n, s_c, s_g, s_w, s_uu, s_w, s_uu);
  if (tid == 0) p.fill[tile] = 0;
}

// dl_init_state: copy (fp32 -> base type) or zero the base and zero every log slot of each tile.
template <int VAR, int DK, int DV, bool BF>
__global__ void __launch_bounds__(256) init_kernel(PoolArgs p, const float* init_base) {
  using BIO = BaseIO<BF>;
  constexpr int CW = (VAR == DL_GDN) ? 1 : DK;
  constexpr int USZ = (VAR == DL_RWKV6) ? 2 : 4;
  const int tid = threadIdx.x;
  const size_t tile = blockIdx.x;
  const size_t L = p.L;
  auto* dst = BIO::tile(p.base, tile * DK * DV);
  const float4* src = init_base ? reinterpret_cast<const float4*>(init_base + tile * DK * DV) : nullptr;
  if (init_base == nullptr || static_cast<const void*>(init_base) != p.base) {
    for (int i = tid; i < DK * DV / 4; i += 256)
      BIO::store(dst, i, src ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f));
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
#define DL_DISPATCH(VAR_, BF_, DK_, DV_, CALL)                             \
  do {                                                                     \
    if ((DK_) == 128 && (DV_) == 128) { CALL(VAR_, BF_, 128, 128); }       \
    else if ((DK_) == 64 && (DV_) == 64) { CALL(VAR_, BF_, 64, 64); }      \
    else if ((DK_) == 128 && (DV_) == 64) { CALL(VAR_, BF_, 128, 64); }    \
    else { CALL(VAR_, BF_, 64, 128); }                                     \
  } while (0)

#define DL_BASES(VAR_, BFI, DK_, DV_, CALL)                                \
  do {                                                                     \
    if (BFI) DL_DISPATCH(VAR_, true, DK_, DV_, CALL);                      \
    else DL_DISPATCH(VAR_, false, DK_, DV_, CALL);                         \
  } while (0)

#define DL_VARIANTS(VARI, BFI, DK_, DV_, CALL)                             \
  do {                                                                     \
    if ((VARI) == DL_GDN) DL_BASES(DL_GDN, BFI, DK_, DV_, CALL);           \
    else if ((VARI) == DL_KDA) DL_BASES(DL_KDA, BFI, DK_, DV_, CALL);      \
    else DL_BASES(DL_RWKV6, BFI, DK_, DV_, CALL);                          \
  } while (0)

hipError_t launch_decode(int variant, bool bf16_base, int dk, int dv, int tiles, const PoolArgs& p,
                         const StepArgs& s, hipStream_t stream) {
  hipError_t err = hipSuccess;
  PoolArgs pa = p;
  StepArgs sa = s;
  void* args[] = {&pa, &sa};
#define CALL_DECODE(V, B, K, D)                                                                        \
  do {                                                                                                 \
    const void* f = reinterpret_cast<const void*>(&decode_kernel<V, K, D, B, 0>);                      \
    int nt = StepGeo<V, K, D, B, 0>::NT;  /* the threads of the kernel picked */                      \
    if (p.L - 1 > 32) {                                                                                \
      f = reinterpret_cast<const void*>(&decode_kernel<V, K, D, B, 64>);                               \
      nt = StepGeo<V, K, D, B, 64>::NT;                                                                \
    } else if (p.L - 1 > StepGeo<V, K, D, B>::PF) {                                                    \
      f = reinterpret_cast<const void*>(&decode_kernel<V, K, D, B, 32>);                               \
      nt = StepGeo<V, K, D, B, 32>::NT;                                                                \
    }                                                                                                  \
    err = hipLaunchKernel(f, dim3(tiles), dim3(nt), args, 0, stream);                                  \
  } while (0)
  DL_VARIANTS(variant, bf16_base, dk, dv, CALL_DECODE);
#undef CALL_DECODE
  return err;
}

hipError_t launch_merge(int variant, bool bf16_base, int dk, int dv, int tiles, const PoolArgs& p,
                        int min_fill, hipStream_t stream) {
  hipError_t err = hipSuccess;
  PoolArgs pa = p;
  int mf = min_fill;
  void* args[] = {&pa, &mf};
#define CALL_MERGE(V, B, K, D)                                                                    \
  err = hipLaunchKernel(reinterpret_cast<const void*>(&merge_kernel<V, K, D, B>), dim3(tiles),    \
                        dim3(StepGeo<V, K, D, B>::NT), args, 0, stream)
  DL_VARIANTS(variant, bf16_base, dk, dv, CALL_MERGE);
#undef CALL_MERGE
  return err;
}

hipError_t launch_init(int variant, bool bf16_base, int dk, int dv, int tiles, const PoolArgs& p,
                       const float* init_base, hipStream_t stream) {
  hipError_t err = hipSuccess;
  PoolArgs pa = p;
  const float* ib = init_base;
  void* args[] = {&pa, &ib};
#define CALL_INIT(V, B, K, D)                                                                     \
  err = hipLaunchKernel(reinterpret_cast<const void*>(&init_kernel<V, K, D, B>), dim3(tiles),     \
                        dim3(256), args, 0, stream)
  DL_VARIANTS(variant, bf16_base, dk, dv, CALL_INIT);
#undef CALL_INIT
  return err;
}

}  // namespace dl

#ifdef DL_TRACE
// Copy the timestamps of workgroups [0, nwg) of both buffers to `host` ([2][nwg][5]
// uint64).  Only in the tracing build.  Returns 0 or the HIP error code.
extern "C" int dl_trace_copy(unsigned long long* host, int nwg) {
  if (nwg < 0 || nwg > 65536) return -1;
  for (int par = 0; par < 2; ++par) {
    const hipError_t e = hipMemcpyFromSymbol(host + (size_t)par * nwg * 5, HIP_SYMBOL(dl::g_trace),
                                             (size_t)nwg * 5 * 8, (size_t)par * 65536 * 5 * 8, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}
#endif
