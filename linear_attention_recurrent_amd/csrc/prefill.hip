// Chunkwise prefill for the GDN delta rule (and its Kaczmarz step size) on gfx950.
//
// dl_prefill runs T prompt tokens of the recurrence
//   S_i = a_i S_{i-1} + k_i u_i^T,   u_i = b_i (v_i - (a_i S_{i-1})^T k_i),   o_i = S_i^T q_i
// for every (sequence, head) tile and leaves S_T in the base.  The Q-Delta,
// Kaczmarz Linear Attention and Gated DeltaNet-2 abstracts (card pages) name
// the chunkwise-parallel (WY) form of delta-rule models; it is derived here for
// one chunk of C tokens starting from state S (g_i = a_1 ... a_i, cumulative
// within the chunk, kept as c_i = log2 g_i):
//   A_ij = b_i (g_i / g_j) (k_i . k_j)   for j < i (strictly lower), T = (I + A)^-1
//   U    = T diag(b) V - T diag(b g) K S                 (rows u_i)
//   O    = diag(g) Q S + (M o Q K^T) U,  M_ij = g_i / g_j for j <= i, else 0
//   S'   = g_C S + (diag(g_C / g) K)^T U
// which is the token-by-token recurrence rewritten: unrolling u_i gives
// (I + A) U = diag(b) (V - diag(g) K S).
//
// Mapping.  One workgroup (4 waves) per tile; wave w owns value columns
// [w dv/4, (w+1) dv/4) of the state, held in MFMA accumulator layout, so the
// dv dimension needs no communication between waves.  Chunk-shared matrices
// (K K^T, Q K^T, T, W = T diag(b g) K) are built once per chunk in LDS.
// Products run on v_mfma_f32_16x16x32_bf16: keys, queries and values are bf16
// already (exact operands); an fp32 operand x is split into bf16 hi + lo with
// x - hi - lo below 2^-17 |x|, and a product of two split operands takes the
// three terms hi*hi + hi*lo + lo*hi, so every product keeps close to fp32
// accuracy while running at the bf16 matrix rate.  The 32 x 32 triangular
// inverse uses fp32 VALU.
//
// MFMA 16x16x32 bf16 lane layout (lane l, n = l % 16, g = l / 16): A[n][8g + s],
// B[8g + s][n] for s < 8; the result holds D[4g + r][n] for r < 4.  Sums over k
// may pair any k order consistently between A and B; the state and U feed the
// B operand straight from accumulator registers with k = {4g + r} u {16 + 4g + r}.
#include "launch.hpp"

namespace dl {
namespace {

using bf16x8 = __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16;
using f32x4 = __attribute__((__vector_size__(4 * sizeof(float)))) float;
using u32x4 = __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t;

constexpr int kChunk = 32;  // tokens per chunk
constexpr int kThreads = 256;

__device__ __forceinline__ f32x4 mma(const bf16x8 a, const bf16x8 b, const f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 u = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 ld_b128(const uint16_t* p) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  return pack8(w.x, w.y, w.z, w.w);
}

// Two groups of four bf16 (8 bytes each) as one operand: slots 0..3, then 4..7.
__device__ __forceinline__ bf16x8 ld_2x64(const uint16_t* p0, const uint16_t* p1) {
  const uint2 a = *reinterpret_cast<const uint2*>(p0);
  const uint2 b = *reinterpret_cast<const uint2*>(p1);
  return pack8(a.x, a.y, b.x, b.y);
}

// Eight bf16 at a stride (a column of a row-major LDS array).
__device__ __forceinline__ bf16x8 ld_col8(const uint16_t* p, int stride) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = uint32_t(p[(2 * i) * stride]) | (uint32_t(p[(2 * i + 1) * stride]) << 16);
  return pack8(w[0], w[1], w[2], w[3]);
}

// Column `n` of a row-major LDS array at the paired token order {4g + s} u {16 + 4g + s}.
__device__ __forceinline__ bf16x8 ld_col_paired(const uint16_t* col, int stride, int g) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint16_t* a = col + (4 * g + 2 * i) * stride;
    const uint16_t* b = col + (16 + 4 * g + 2 * i) * stride;
    w[i] = uint32_t(a[0]) | (uint32_t(a[stride]) << 16);
    w[2 + i] = uint32_t(b[0]) | (uint32_t(b[stride]) << 16);
  }
  return pack8(w[0], w[1], w[2], w[3]);
}

// fp32 -> bf16 hi + lo (bit patterns).
__device__ __forceinline__ void split(float x, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_rne(x);
  lo = f32_to_bf16_rne(x - bf16_to_f32(hi));
}

// Two accumulator blocks (4 values each, k = 4g + r and 16 + 4g + r) as split B operands.
__device__ __forceinline__ void split_pair(const float (&x0)[4], const float (&x1)[4], bf16x8& hi, bf16x8& lo) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    split(x0[r], h[r], l[r]);
    split(x1[r], h[4 + r], l[4 + r]);
  }
  hi = pack8(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
  lo = pack8(l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16));
}

template <bool BF>
__device__ __forceinline__ float ld_base(const void* base, size_t i) {
  if constexpr (BF) return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
  else return static_cast<const float*>(base)[i];
}
template <bool BF>
__device__ __forceinline__ void st_base(void* base, size_t i, float x) {
  if constexpr (BF) static_cast<uint16_t*>(base)[i] = static_cast<uint16_t>(f32_to_bf16_rne(x));
  else static_cast<float*>(base)[i] = x;
}

template <int DK, int DV>
struct PrefillLds {
  static constexpr int C = kChunk;
  static constexpr int KS = DK + 8;  // bf16 row stride of the K, Q and W arrays (16-byte pad)
  static constexpr int VS = DV + 8;  // bf16 row stride of V
  static constexpr int MS = C + 1;   // fp32 row stride of the C x C matrices
  static constexpr int BS = C + 8;   // bf16 row stride of the split C x C matrices
  uint16_t k[C * KS];
  uint16_t q[C * KS];
  uint16_t v[C * VS];
  uint16_t wh[C * KS], wl[C * KS];  // W = T diag(b g) K, split
  float g[C * MS];                   // K K^T, then A (strictly lower part)
  float p[C * MS];                   // Q K^T; later 16 x 17 scratch for the off-diagonal block of T
  float t[C * MS];                   // T = (I + A)^-1
  uint16_t t1h[C * BS], t1l[C * BS];  // T diag(b)
  uint16_t t2h[C * BS], t2l[C * BS];  // T diag(b g)
  uint16_t pmh[C * BS], pml[C * BS];  // M o Q K^T
  float c[C];                         // cumulative log2 decay within the chunk
  float gam[C];                       // 2^c
  float beta[C];                      // step size (0 for tokens past the end)
  float braw[C];                      // beta or eta as given
  float knorm[C];                     // ||k||^2 (Kaczmarz step size)
};

template <int DK, int DV, bool BF>
__global__ void __launch_bounds__(kThreads) prefill_kernel(PoolArgs pa, PrefillArgs a) {
  constexpr int C = kChunk;
  constexpr int CW = DV / 4;    // value columns per wave
  constexpr int NCB = CW / 16;  // 16-column blocks per wave
  constexpr int NKB = DK / 16;  // 16-channel blocks
  constexpr int NKP = DK / 32;  // pairs of channel blocks (one MFMA k-step each)
  using Lds = PrefillLds<DK, DV>;
  constexpr int KS = Lds::KS, VS = Lds::VS, MS = Lds::MS, BS = Lds::BS;
  static_assert(NCB >= 1 && NKP >= 1, "head sizes 64 or 128");
  __shared__ __align__(16) Lds sh;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int tile = blockIdx.x;
  const int H = pa.heads, T = a.tokens;
  const size_t bseq = static_cast<size_t>(tile / H), h = static_cast<size_t>(tile % H);
  const int col0 = wave * CW;

  // The state columns of this wave: S[kb][cb][r] = S(16 kb + 4 lg + r, col0 + 16 cb + ln).
  float S[NKB][NCB][4];
  const size_t tbase = static_cast<size_t>(tile) * DK * DV;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S[kb][cb][r] = ld_base<BF>(pa.base, tbase + size_t(16 * kb + 4 * lg + r) * DV + col0 + 16 * cb + ln);

  const bool kla = a.eta != nullptr;
  for (int t0 = 0; t0 < T; t0 += C) {
    __syncthreads();  // every wave is done with the previous chunk's LDS arrays

    // ---- 1. this chunk's rows of K, Q, V (zeros past the end); ||k||^2; decays
    auto row_ptr = [&](const uint16_t* x, int t, int d) {
      return x + ((bseq * T + t) * H + h) * d;
    };
#pragma unroll
    for (int i = 0; i < C * DK / 8 / kThreads; ++i) {
      const int pc = tid + i * kThreads, row = pc / (DK / 8), seg = pc % (DK / 8);
      const bool ok = t0 + row < T;
      uint4 kw = make_uint4(0, 0, 0, 0), qw = kw;
      if (ok) {
        kw = reinterpret_cast<const uint4*>(row_ptr(a.k, t0 + row, DK))[seg];
        qw = reinterpret_cast<const uint4*>(row_ptr(a.q, t0 + row, DK))[seg];
      }
      *reinterpret_cast<uint4*>(&sh.k[row * KS + seg * 8]) = kw;
      *reinterpret_cast<uint4*>(&sh.q[row * KS + seg * 8]) = qw;
      if (kla) {
        float f[8];
        unpack8(kw, f);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
        ss = group_sum<DK / 8>(ss);
        if (seg == 0) sh.knorm[row] = ss;
      }
    }
#pragma unroll
    for (int i = 0; i < C * DV / 8 / kThreads; ++i) {
      const int pc = tid + i * kThreads, row = pc / (DV / 8), seg = pc % (DV / 8);
      uint4 vw = make_uint4(0, 0, 0, 0);
      if (t0 + row < T) vw = reinterpret_cast<const uint4*>(row_ptr(a.v, t0 + row, DV))[seg];
      *reinterpret_cast<uint4*>(&sh.v[row * VS + seg * 8]) = vw;
    }
    if (wave == 3) {
      // lanes 0..31: one token each; inclusive prefix sum of the clamped log2 decays
      const int t = t0 + lane;
      const bool ok = lane < C && t < T;
      const size_t si = (bseq * T + (ok ? t : 0)) * H + h;
      float l2 = ok ? step_log2_decay(a.decay[si]) : 0.f;
      const float bt = ok ? (kla ? a.eta[si] : a.beta[si]) : 0.f;
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) {
        const float y = __shfl_up(l2, off, 64);
        if (lane >= off) l2 += y;
      }
      if (lane < C) {
        sh.c[lane] = l2;
        sh.gam[lane] = exp2f(l2);
        sh.braw[lane] = bt;
      }
    }
    __syncthreads();

    // ---- 2. G = K K^T and P = Q K^T on the lower blocks (waves 0..2); step sizes (wave 3)
    if (wave < 3) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int blk = 2 * wave + e;  // 0..2: G blocks (0,0), (1,0), (1,1); 3..5: the same of P
        const int sub = blk % 3;
        const int ib = sub == 0 ? 0 : 1, jb = sub == 2 ? 1 : 0;
        const uint16_t* xa = blk < 3 ? sh.k : sh.q;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk)
          acc = mma(ld_b128(&xa[(16 * ib + ln) * KS + 32 * kk + 8 * lg]),
                    ld_b128(&sh.k[(16 * jb + ln) * KS + 32 * kk + 8 * lg]), acc);
        float* dst = blk < 3 ? sh.g : sh.p;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * ib + 4 * lg + r) * MS + 16 * jb + ln] = acc[r];
      }
    } else if (lane < C) {
      const bool ok = t0 + lane < T;
      sh.beta[lane] = !ok ? 0.f : kla ? sh.braw[lane] / (sh.knorm[lane] + a.eps) : sh.braw[lane];
    }
    __syncthreads();

    // ---- 3. A = strictly lower b_i 2^(c_i - c_j) G_ij (in place); M o P split; T's upper block = 0
    for (int e = tid; e < C * C; e += kThreads) {
      const int i = e / C, j = e % C;
      if (j < i) sh.g[i * MS + j] *= sh.beta[i] * exp2f(sh.c[i] - sh.c[j]);
      const float pm = j <= i ? exp2f(sh.c[i] - sh.c[j]) * sh.p[i * MS + j] : 0.f;
      uint32_t hi, lo;
      split(pm, hi, lo);
      sh.pmh[i * BS + j] = static_cast<uint16_t>(hi);
      sh.pml[i * BS + j] = static_cast<uint16_t>(lo);
      if (i < 16 && j >= 16) sh.t[i * MS + j] = 0.f;
    }
    __syncthreads();

    // ---- 4. diagonal 16 x 16 blocks of T by forward substitution (lane j: column j)
    if (wave < 2 && lane < 16) {
      const int o = 16 * wave;
      float x[16];
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        float s = m == lane ? 1.f : 0.f;
#pragma unroll
        for (int pp = 0; pp < m; ++pp) s = fmaf(-sh.g[(o + m) * MS + o + pp], x[pp], s);
        x[m] = s;
      }
#pragma unroll
      for (int m = 0; m < 16; ++m) sh.t[(o + m) * MS + o + lane] = x[m];
    }
    __syncthreads();

    // ---- 5. off-diagonal block: T_10 = -T_11 (A_10 T_00)
    float* xs = sh.p;  // P is no longer needed
    {
      const int i = tid >> 4, j = tid & 15;
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) s = fmaf(sh.g[(16 + i) * MS + m], sh.t[m * MS + j], s);
      xs[i * 17 + j] = s;
      __syncthreads();
      float y = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) y = fmaf(sh.t[(16 + i) * MS + 16 + m], xs[m * 17 + j], y);
      sh.t[(16 + i) * MS + j] = -y;
    }
    __syncthreads();

    // ---- 6. T diag(b) and T diag(b g), split
    for (int e = tid; e < C * C; e += kThreads) {
      const int i = e / C, j = e % C;
      const float t1 = sh.t[i * MS + j] * sh.beta[j];
      uint32_t hi, lo;
      split(t1, hi, lo);
      sh.t1h[i * BS + j] = static_cast<uint16_t>(hi);
      sh.t1l[i * BS + j] = static_cast<uint16_t>(lo);
      split(t1 * sh.gam[j], hi, lo);
      sh.t2h[i * BS + j] = static_cast<uint16_t>(hi);
      sh.t2l[i * BS + j] = static_cast<uint16_t>(lo);
    }
    __syncthreads();

    // ---- 7. W = T diag(b g) K into LDS (blocks shared out over the waves); this wave's T diag(b) V
#pragma unroll
    for (int e = 0; e < NKB / 2; ++e) {
      const int blk = wave + 4 * e;  // 2 * NKB blocks: (ib, cb) = (blk / NKB, blk % NKB)
      const int ib = blk / NKB, cb = blk % NKB;
      const bf16x8 kb8 = ld_col8(&sh.k[(8 * lg) * KS + 16 * cb + ln], KS);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mma(ld_b128(&sh.t2h[(16 * ib + ln) * BS + 8 * lg]), kb8, acc);
      acc = mma(ld_b128(&sh.t2l[(16 * ib + ln) * BS + 8 * lg]), kb8, acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t hi, lo;
        split(acc[r], hi, lo);
        sh.wh[(16 * ib + 4 * lg + r) * KS + 16 * cb + ln] = static_cast<uint16_t>(hi);
        sh.wl[(16 * ib + 4 * lg + r) * KS + 16 * cb + ln] = static_cast<uint16_t>(lo);
      }
    }
    float U[2][NCB][4];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const bf16x8 vb8 = ld_col8(&sh.v[(8 * lg) * VS + col0 + 16 * cb + ln], VS);
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma(ld_b128(&sh.t1h[(16 * ib + ln) * BS + 8 * lg]), vb8, acc);
        acc = mma(ld_b128(&sh.t1l[(16 * ib + ln) * BS + 8 * lg]), vb8, acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) U[ib][cb][r] = acc[r];
      }
    }
    __syncthreads();

    // ---- 8. U = T diag(b) V - W S, and diag(g) Q S, with S split once
    bf16x8 shi[NKP][NCB], slo[NKP][NCB];
#pragma unroll
    for (int kp = 0; kp < NKP; ++kp)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) split_pair(S[2 * kp][cb], S[2 * kp + 1][cb], shi[kp][cb], slo[kp][cb]);
    float O[2][NCB][4];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      f32x4 ws[NCB], qs[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        ws[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
        qs[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kp = 0; kp < NKP; ++kp) {
        const int rowk = (16 * ib + ln) * KS + 32 * kp + 4 * lg;
        const bf16x8 wah = ld_2x64(&sh.wh[rowk], &sh.wh[rowk + 16]);
        const bf16x8 wal = ld_2x64(&sh.wl[rowk], &sh.wl[rowk + 16]);
        const bf16x8 qa = ld_2x64(&sh.q[rowk], &sh.q[rowk + 16]);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          ws[cb] = mma(wah, shi[kp][cb], ws[cb]);
          ws[cb] = mma(wah, slo[kp][cb], ws[cb]);
          ws[cb] = mma(wal, shi[kp][cb], ws[cb]);
          qs[cb] = mma(qa, shi[kp][cb], qs[cb]);
          qs[cb] = mma(qa, slo[kp][cb], qs[cb]);
        }
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          U[ib][cb][r] -= ws[cb][r];
          O[ib][cb][r] = sh.gam[16 * ib + 4 * lg + r] * qs[cb][r];
        }
    }

    // ---- 9. O += (M o Q K^T) U; write the outputs
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      bf16x8 uhi, ulo;
      split_pair(U[0][cb], U[1][cb], uhi, ulo);
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        const int rowp = (16 * ib + ln) * BS + 4 * lg;
        const bf16x8 pah = ld_2x64(&sh.pmh[rowp], &sh.pmh[rowp + 16]);
        const bf16x8 pal = ld_2x64(&sh.pml[rowp], &sh.pml[rowp + 16]);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma(pah, uhi, acc);
        acc = mma(pah, ulo, acc);
        acc = mma(pal, uhi, acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + 16 * ib + 4 * lg + r;
          if (t < T) a.out[((bseq * T + t) * H + h) * DV + col0 + 16 * cb + ln] = O[ib][cb][r] + acc[r];
        }
      }
    }

    // ---- 10. S = g_C S + K^T (diag(2^(c_C - c_j)) U)
    const float gC = sh.gam[C - 1], cC = sh.c[C - 1];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float f = exp2f(cC - sh.c[16 * ib + 4 * lg + r]);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) U[ib][cb][r] *= f;
      }
    bf16x8 u2hi[NCB], u2lo[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) split_pair(U[0][cb], U[1][cb], u2hi[cb], u2lo[cb]);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const bf16x8 ka = ld_col_paired(&sh.k[16 * kb + ln], KS, lg);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        f32x4 acc = {gC * S[kb][cb][0], gC * S[kb][cb][1], gC * S[kb][cb][2], gC * S[kb][cb][3]};
        acc = mma(ka, u2hi[cb], acc);
        acc = mma(ka, u2lo[cb], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) S[kb][cb][r] = acc[r];
      }
    }
  }

#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        st_base<BF>(pa.base, tbase + size_t(16 * kb + 4 * lg + r) * DV + col0 + 16 * cb + ln, S[kb][cb][r]);
}

}  // namespace

hipError_t launch_prefill(bool bf16_base, int dk, int dv, int tiles, const PoolArgs& p, const PrefillArgs& a,
                          hipStream_t stream) {
#define DL_PREFILL(BF_, DK_, DV_) \
  prefill_kernel<DK_, DV_, BF_><<<tiles, kThreads, 0, stream>>>(p, a)
#define DL_PREFILL_SHAPES(BF_)                                  \
  do {                                                          \
    if (dk == 128 && dv == 128) DL_PREFILL(BF_, 128, 128);      \
    else if (dk == 64 && dv == 64) DL_PREFILL(BF_, 64, 64);     \
    else if (dk == 128 && dv == 64) DL_PREFILL(BF_, 128, 64);   \
    else DL_PREFILL(BF_, 64, 128);                              \
  } while (0)
  if (bf16_base) DL_PREFILL_SHAPES(true);
  else DL_PREFILL_SHAPES(false);
#undef DL_PREFILL_SHAPES
#undef DL_PREFILL
  return hipGetLastError();
}

}  // namespace dl
