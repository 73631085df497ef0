// Chunkwise prefill on gfx950: the GDN delta rule (and its Kaczmarz step size)
// below, KDA and RWKV6 further down.
//
// For GDN, dl_prefill runs T prompt tokens of the recurrence
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
// Mapping.  One workgroup per tile (eight waves for dv = 128, else four); wave w owns
// value columns [w dv/W, (w+1) dv/W) of the state (W waves), held in MFMA accumulator
// layout, so the dv dimension needs no communication between waves.  Chunk-shared matrices
// (K K^T, Q K^T, T diag(b)) are built once per chunk in LDS.  The state enters U as
// U = T diag(b) (V - diag(g) X) with X = K S: X takes the exact bf16 keys against the
// split state, R = V - diag(g) X is formed in fp32 where X sits in registers, and R
// feeds T diag(b) R, so no C x dk product of T with K is formed or staged.
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
// B operand straight from accumulator registers with k = {4g + r} u {16 + 4g + r}
// (so does R, over tokens).
// Every array is stored in token rows.  Rows that are the A operand against such an
// accumulator-layout B operand keep each 32-element block in that k order (kperm), so
// the operand is one 16-byte read; where tokens run along an operand's k index (K^T and
// its decay-scaled copies in the state update, V) the rows are read through
// ds_read_b64_tr_b16.  Row strides follow gfx950's banks (64 banks of 4 bytes): 8 mod 16
// words for 16-byte and transposing reads.
#include "launch.hpp"

namespace dl {
namespace {

using bf16x8 = __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16;
using f32x4 = __attribute__((__vector_size__(4 * sizeof(float)))) float;
using u32x4 = __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t;
using bf16x2 = __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16;

constexpr int kChunk = 32;  // tokens per chunk
constexpr int kThreads = 256;  // RWKV6 workgroup

// max(log2 d, -126) with the bare v_log_f32: for d not below the smallest normal float the
// same value as log2f (which only adds a rescaling for denormal inputs), and for smaller d
// the same clamped value.
__device__ __forceinline__ float chunk_log2_decay(float d) {
  return fmaxf(__builtin_amdgcn_logf(d), kMinLog2Decay);
}

// 2^x with the bare hardware instruction (about 1 ulp).  Every argument here is a
// difference of cumulative log2 decays; results below 2^-126 (the normal range)
// stand for products of decays that are negligible next to the other terms.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

// ds_read_b64_tr_b16: each lane names 4 consecutive bf16 (8 bytes); within each group of
// 16 lanes, lane l receives element l % 4 of the reads of lanes l / 4 + 4 s, s = 0..3.
// With lane j of a group reading row r0 + j / 4 at column c0 + 4 (j % 4) of a row-major
// bf16 array, lane l gets rows r0 .. r0 + 3 of column c0 + l: a 4 x 16 block read
// transposed, which is half of an MFMA operand whose k index runs along the rows.
typedef short short4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 ld_tr4(const uint16_t* p) {
  const short4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p));
  return __builtin_bit_cast(uint2, r);
}
// An operand whose k slots 0..3 and 4..7 are rows r0.. and r1.. of column c0 + (lane % 16)
// of a row-major bf16 array with row stride rs: lane j of the group passes its own
// row and column offsets.
__device__ __forceinline__ bf16x8 ld_tr8(const uint16_t* base, int rs, int r0, int r1, int c0, int j) {
  const int off = (j >> 2) * rs + c0 + 4 * (j & 3);
  const uint2 a = ld_tr4(base + r0 * rs + off), b = ld_tr4(base + r1 * rs + off);
  return pack8(a.x, a.y, b.x, b.y);
}

// The same with this lane's own column (already mapped to storage order).
__device__ __forceinline__ bf16x8 ld_tr8_at(const uint16_t* base, int rs, int r0, int r1, int col, int j) {
  const int off = (j >> 2) * rs + col;
  const uint2 a = ld_tr4(base + r0 * rs + off), b = ld_tr4(base + r1 * rs + off);
  return pack8(a.x, a.y, b.x, b.y);
}

// Rows that are the A operand of a product whose B operand comes from accumulator
// registers (k = {4g + r} u {16 + 4g + r}) keep each 32-element block in that k order:
// logical elements 4g .. 4g + 3 and 16 + 4g .. 16 + 4g + 3 side by side, so the operand
// is one 16-byte read (two 8-byte reads of one lane, merged by the compiler into
// ds_read2_b64, cost several times as much on gfx950).  kperm(e) is the storage position
// of logical element e; groups of 4 stay contiguous.
__device__ __forceinline__ int kperm(int e) { return (e & ~31) | ((e & 12) << 1) | ((e & 16) >> 2) | (e & 3); }
// 8 logical elements e0 .. e0 + 7 (e0 a multiple of 8) of such a row.
__device__ __forceinline__ void st_kperm8(uint16_t* row, int e0, uint4 w) {
  *reinterpret_cast<uint2*>(&row[kperm(e0)]) = make_uint2(w.x, w.y);
  *reinterpret_cast<uint2*>(&row[kperm(e0 + 4)]) = make_uint2(w.z, w.w);
}

// Inclusive prefix sum over lanes 0..31 of a wave with DPP moves: shifts by 1, 2, 4 and 8
// within each row of 16 lanes, then row 0's total (lane 15) added to row 1.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_or_zero(float v) {  // lanes with no source lane get 0
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf, false));
}
__device__ __forceinline__ float scan32(float x) {
  x += dpp_or_zero<0x111, 0xf>(x);  // row_shr:1
  x += dpp_or_zero<0x112, 0xf>(x);  // row_shr:2
  x += dpp_or_zero<0x114, 0xf>(x);  // row_shr:4
  x += dpp_or_zero<0x118, 0xf>(x);  // row_shr:8
  x += dpp_or_zero<0x142, 0xa>(x);  // row_bcast:15, into rows 1 and 3
  return x;
}

// Two fp32 values rounded to bf16 (to nearest, ties to even; one v_cvt_pk_bf16_f32)
// and packed, a in the low half.
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// A packed bf16 pair held in a register.  Written as a literal, the pair (-1, 0) is
// encoded by the compiler as the inline constant -1.0, which v_dot2c_f32_bf16 reads as
// the pair (0, -1); the empty asm keeps the bits in an SGPR so the operand is the pair
// as written.
__device__ __forceinline__ bf16x2 pair_in_reg(uint32_t bits) {
  asm("" : "+s"(bits));
  return __builtin_bit_cast(bf16x2, bits);
}

// x - (the bf16 number in the low, or high, half of h) in one v_dot2c_f32_bf16 against
// (-1, 0), or (0, -1): the product is exact and, when that half is x rounded to bf16,
// so is the difference.  (Finite operands: the other half enters multiplied by 0.)
__device__ __forceinline__ float rem_lo(uint32_t h, float x) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, h), pair_in_reg(0x0000bf80u), x, false);
}
__device__ __forceinline__ float rem_hi(uint32_t h, float x) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, h), pair_in_reg(0xbf800000u), x, false);
}

// fp32 -> bf16 hi + lo for two values at once (packed pairs); x - hi is exact in fp32.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = cvt2(a, b);
  lo = cvt2(rem_lo(hi, a), rem_hi(hi, b));
}

// fp32 -> bf16 hi + mid + lo for two values at once: x - hi - mid - lo is below 2^-26 |x|.
// Used for the decay-weighted key/query products, whose sums over channels cancel.
__device__ __forceinline__ void split3(float a, float b, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = cvt2(a, b);
  const float ra = rem_lo(hi, a), rb = rem_hi(hi, b);
  mid = cvt2(ra, rb);
  lo = cvt2(rem_lo(mid, ra), rem_hi(mid, rb));
}

// sum of the products of two three-way split operands, terms down to 2^-16 of the
// leading one: hi.hi + hi.mid + mid.hi + hi.lo + mid.mid + lo.hi.
__device__ __forceinline__ f32x4 mma3(const bf16x8 (&x)[3], const bf16x8 (&y)[3], f32x4 acc) {
  acc = mma(x[0], y[0], acc);
  acc = mma(x[0], y[1], acc);
  acc = mma(x[1], y[0], acc);
  acc = mma(x[0], y[2], acc);
  acc = mma(x[1], y[1], acc);
  acc = mma(x[2], y[0], acc);
  return acc;
}

// Two accumulator blocks (4 values each, k = 4g + r and 16 + 4g + r) as split B operands.
__device__ __forceinline__ void split_pair(const float (&x0)[4], const float (&x1)[4], bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
  split2(x0[0], x0[1], h[0], l[0]);
  split2(x0[2], x0[3], h[1], l[1]);
  split2(x1[0], x1[1], h[2], l[2]);
  split2(x1[2], x1[3], h[3], l[3]);
  hi = pack8(h[0], h[1], h[2], h[3]);
  lo = pack8(l[0], l[1], l[2], l[3]);
}

// One state element of a tile through a buffer resource over that tile: the
// per-lane part of the offset is one VGPR and the rest an immediate, so the 64
// addresses of a lane's state elements are never materialised as registers.
template <bool BF>
__device__ __forceinline__ float ld_base(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  if constexpr (BF) return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
  else return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
template <bool BF>
__device__ __forceinline__ void st_base(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, float x) {
  if constexpr (BF)
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(f32_to_bf16_rne(x)), r, voff, soff, 0);
  else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, voff, soff, 0);
}


// x_i -= g_i' y for i < N (N <= 4), where g' is g as held by lane P of this lane's row of
// 16 lanes: one v_fmac_f32_dpp each, with a row_newbcast source (the broadcast and the
// negation are operand modifiers).  The leading s_nop 1 gives the two wait states that a
// DPP read of a VGPR needs after a VALU write of it (the compiler does not see into the
// asm to add them); inside the block no instruction writes a DPP source.
// one FMA: x operand i, g operand j, y operand k, P operand l
#define DL_FNMA_BC(i, j, k, l) \
  "v_fmac_f32_dpp %" #i ", -%" #j ", %" #k " row_newbcast:%" #l " row_mask:0xf bank_mask:0xf\n\t"
template <int P, int N>
__device__ __forceinline__ void fnma_row_bcast(float* x, const float* g, float y) {
  static_assert(N >= 1 && N <= 4, "one to four rows");
  if constexpr (N == 4)
    asm volatile("s_nop 1\n\t" DL_FNMA_BC(0, 4, 8, 9) DL_FNMA_BC(1, 5, 8, 9) DL_FNMA_BC(2, 6, 8, 9)
                     DL_FNMA_BC(3, 7, 8, 9)
                 : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3])
                 : "v"(g[0]), "v"(g[1]), "v"(g[2]), "v"(g[3]), "v"(y), "n"(P));
  else if constexpr (N == 3)
    asm volatile("s_nop 1\n\t" DL_FNMA_BC(0, 3, 6, 7) DL_FNMA_BC(1, 4, 6, 7) DL_FNMA_BC(2, 5, 6, 7)
                 : "+v"(x[0]), "+v"(x[1]), "+v"(x[2])
                 : "v"(g[0]), "v"(g[1]), "v"(g[2]), "v"(y), "n"(P));
  else if constexpr (N == 2)
    asm volatile("s_nop 1\n\t" DL_FNMA_BC(0, 2, 4, 5) DL_FNMA_BC(1, 3, 4, 5)
                 : "+v"(x[0]), "+v"(x[1])
                 : "v"(g[0]), "v"(g[1]), "v"(y), "n"(P));
  else
    asm volatile("s_nop 1\n\t" DL_FNMA_BC(0, 1, 2, 3) : "+v"(x[0]) : "v"(g[0]), "v"(y), "n"(P));
}
#undef DL_FNMA_BC

// Forward substitution steps P .. BS - 2 for one BS x BS unit lower block, one column
// per lane: once x_P is final, x_m -= A_mP x_P for every later row m (right-looking, so
// the dependent chain is one FMA per row); A_mP is this lane's gc[m] as held by lane P.
template <int BS, int P, int M = P + 1>
__device__ __forceinline__ void substitute_from(float (&x)[BS], const float (&gc)[BS]) {
  if constexpr (P < BS - 1) {
    constexpr int N = BS - M < 4 ? BS - M : 4;
    fnma_row_bcast<P, N>(&x[M], &gc[M], x[P]);
    if constexpr (M + N < BS) substitute_from<BS, P, M + N>(x, gc);
    else substitute_from<BS, P + 1>(x, gc);
  }
}

// Orders one wave's LDS accesses: the wave's earlier LDS writes have completed before
// any later access (other lanes of the wave read what these lanes wrote).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// T diag(b) for T = (I + A)^-1 and a 32 x 32 strictly lower A (fp32 in LDS, row stride
// MS), split (hi, lo) into th and tl in k order (row stride TB): the A operand of
// T diag(b) R.  Wave 0 inverts the two diagonal 16 x 16 blocks into t (fp32): the four
// diagonal 8 x 8 blocks by forward substitution (one per row of 16 lanes; lane: column),
// then in each 16 x 16 block T_10 = -T_11 (A_10 T_00) over 8 x 8 blocks, two entries a
// lane.  Then, on the first 256 threads, one entry each of Y = A_10 T_00 for the 16 x 16
// blocks, while 256 threads (the same ones for a workgroup of 256, the next ones for 512)
// split the diagonal blocks of T diag(b), two adjacent columns each; then
// T_10 = -T_11 Y, one entry a thread, times b and split.  The upper right blocks of th
// and tl must already be zero.  xs: 16 x 17 floats of scratch.  Called by the whole
// workgroup (it synchronises); returns after a barrier.
template <int MS, int TB, int NT>
__device__ __forceinline__ void invert_unit_lower32(const float* g, float* t, float* xs, const float* b,
                                                    uint16_t* th, uint16_t* tl, int tid) {
  static_assert(NT == 256 || NT == 512, "workgroup of 256 or 512 threads");
  static_assert(MS % 4 == 0, "16-byte row reads");
  if (tid < 64) {
    {  // the 8 x 8 block at o8 (lanes 8..15 of a row repeat columns 0..7 and store nothing)
      const int o8 = 8 * (tid >> 4);
      int col = tid & 7;
      asm volatile("" : "+v"(col));  // keeps the 8 (m == col) selects as selects
      float gc[8], x[8];
      gc[0] = 0.f;
#pragma unroll
      for (int m = 1; m < 8; ++m) gc[m] = g[(o8 + m) * MS + o8 + col];  // A(o8 + m, o8 + col)
#pragma unroll
      for (int m = 0; m < 8; ++m) x[m] = m == col ? 1.f : 0.f;
      substitute_from<8, 0>(x, gc);
      if ((tid & 15) < 8) {
#pragma unroll
        for (int m = 0; m < 8; ++m) t[(o8 + m) * MS + o8 + col] = x[m];
      }
    }
    // 16 x 16 block o: lane (i, columns j, j + 1) of Y8 = A_10 T_00 and T_10 = -T_11 Y8,
    // where the blocks are 8 x 8; the upper right 8 x 8 block of T is zero
    const int o = 16 * (tid >> 5), i = (tid >> 2) & 7, j = 2 * (tid & 3);
    *reinterpret_cast<float2*>(&t[(o + i) * MS + o + 8 + j]) = make_float2(0.f, 0.f);
    wave_lds_sync();
    {
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(&g[(o + 8 + i) * MS + o]);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(&g[(o + 8 + i) * MS + o + 4]);
      float y0 = 0.f, y1 = 0.f;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float am = m < 4 ? a0[m] : a1[m - 4];
        const float2 d = *reinterpret_cast<const float2*>(&t[(o + m) * MS + o + j]);
        y0 = fmaf(am, d.x, y0);
        y1 = fmaf(am, d.y, y1);
      }
      *reinterpret_cast<float2*>(&xs[((o >> 1) + i) * 8 + j]) = make_float2(y0, y1);
    }
    wave_lds_sync();
    {
      const f32x4 d0 = *reinterpret_cast<const f32x4*>(&t[(o + 8 + i) * MS + o + 8]);
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(&t[(o + 8 + i) * MS + o + 12]);
      float z0 = 0.f, z1 = 0.f;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float dm = m < 4 ? d0[m] : d1[m - 4];
        const float2 y = *reinterpret_cast<const float2*>(&xs[((o >> 1) + m) * 8 + j]);
        z0 = fmaf(dm, y.x, z0);
        z1 = fmaf(dm, y.y, z1);
      }
      *reinterpret_cast<float2*>(&t[(o + 8 + i) * MS + o + j]) = make_float2(-z0, -z1);
    }
  }
  __syncthreads();
  // rows of A and T are read 4 at a time (MS is a multiple of 4); the sums run over m in order
  const int i = (tid >> 4) & 15, j = tid & 15;
  if (tid < 256) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(&g[(16 + i) * MS + 4 * q]);
#pragma unroll
      for (int u = 0; u < 4; ++u) s = fmaf(a4[u], t[(4 * q + u) * MS + j], s);
    }
    xs[i * 17 + j] = s;
  }
  {
    const int sid = NT == 512 ? tid - 256 : tid;  // diagonal block o / 16, row r, columns c, c + 1
    if (sid >= 0) {
      const int o = (sid >> 7) * 16, r = (sid >> 3) & 15, c = 2 * (sid & 7);
      const float2 tv = *reinterpret_cast<const float2*>(&t[(o + r) * MS + o + c]);
      uint32_t hi, lo;
      split2(tv.x * b[o + c], tv.y * b[o + c + 1], hi, lo);
      *reinterpret_cast<uint32_t*>(&th[(o + r) * TB + kperm(o + c)]) = hi;
      *reinterpret_cast<uint32_t*>(&tl[(o + r) * TB + kperm(o + c)]) = lo;
    }
  }
  __syncthreads();
  if (tid < 256) {
    float y = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 t4 = *reinterpret_cast<const f32x4*>(&t[(16 + i) * MS + 16 + 4 * q]);
#pragma unroll
      for (int u = 0; u < 4; ++u) y = fmaf(t4[u], xs[(4 * q + u) * 17 + j], y);
    }
    uint32_t hi, lo;
    split2(-y * b[j], 0.f, hi, lo);
    th[(16 + i) * TB + kperm(j)] = static_cast<uint16_t>(hi);
    tl[(16 + i) * TB + kperm(j)] = static_cast<uint16_t>(lo);
  }
  __syncthreads();
}

// Rows t0 .. t0 + C - 1 of one (sequence, head) of a [batch][T][heads][row] input as a
// buffer resource that ends after the prompt's last row: rows past it read as zeros, with
// no branch and no 64-bit address arithmetic per load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rows(const void* x, size_t bseq, size_t h, int T, int H,
                                                              int t0, int bytes_per_row) {
  const int rows = T - t0 < kChunk ? T - t0 : kChunk;
  return make_rsrc(static_cast<const char*>(x) + ((bseq * T + t0) * H + h) * bytes_per_row,
                   static_cast<uint32_t>(rows * H * bytes_per_row));
}

// Output rows t0 .. t0 + C - 1 of one sequence as a buffer resource that covers only
// the rows the prompt has: a store to a row past its end lies outside the resource
// and is dropped, so the stores need no branch and one VGPR offset each.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rows(float* out, size_t bseq, int T, int H, int DV, int t0,
                                                            int C) {
  const int rows = T - t0 < C ? T - t0 : C;
  return make_rsrc(out + (bseq * T + t0) * H * DV, rows * H * DV * 4);
}
// Four consecutive columns of one output row in one 16-byte store.  The output products
// are formed transposed (the operands of the MFMA swapped), so a lane's four accumulator
// rows are four adjacent value columns of a single token.
__device__ __forceinline__ void st_out4(__amdgpu_buffer_rsrc_t r, uint32_t off, const f32x4 x) {
  using u32x4 = __attribute__((ext_vector_type(4))) unsigned int;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, 0);
}

template <int DK, int DV>
struct PrefillLds {
  static constexpr int C = kChunk;
  // Row strides (bf16) of 8 mod 16 words: 16-byte and transposing reads of 16 consecutive
  // rows then fall on distinct banks (gfx950: 64 banks of 4 bytes).
  static constexpr int KS = DK + 16;  // K and Q (k order, kperm)
  static constexpr int VS = DV + 16;  // V
  static constexpr int TB = C + 16;   // split C x C matrices
  static constexpr int MS = C + 4;    // fp32 row stride of the C x C matrices (16-byte rows)
  float c[C];      // cumulative log2 decay within the chunk
  float gam[C];    // 2^c
  float beta[C];   // step size (0 for tokens past the end)
  float braw[C];   // beta or eta as given
  float g[C * MS];  // K K^T, then A (strictly lower part)
  union {
    float p[C * MS];  // Q K^T
    float t[C * MS];  // then the diagonal blocks of T = (I + A)^-1
  };
  float xs[16 * 17];     // scratch for the off-diagonal block of T
  uint16_t t1h[C * TB];  // T diag(b) (hi part, k order; upper right block zero)
  uint16_t t1l[C * TB];
  uint16_t pmh[C * TB], pml[C * TB];  // M o Q K^T, k order
  uint16_t k[C * KS];  // K, token rows, k order
  uint16_t q[C * KS];  // Q, token rows, k order
  uint16_t v[C * VS];  // V, token rows
};

// Threads of a GDN workgroup: eight waves of 16 value columns each for dv = 128 (up to
// 128 VGPRs, so four waves share each SIMD: two workgroups per CU), else four.
template <int DV>
constexpr int gdn_threads() { return DV == 128 ? 512 : 256; }

template <int DK, int DV, bool BF>
__global__ void __launch_bounds__(gdn_threads<DV>(), gdn_threads<DV>() == 512 ? 4 : 2) prefill_kernel(PoolArgs pa, PrefillArgs a) {
  constexpr int C = kChunk;
  constexpr int NT = gdn_threads<DV>(), NWV = NT / 64;  // threads, waves
  constexpr int CW = DV / NWV;  // value columns per wave
  constexpr int NCB = CW / 16;  // 16-column blocks per wave
  constexpr int NKB = DK / 16;  // 16-channel blocks
  constexpr int NKP = DK / 32;  // pairs of channel blocks (one MFMA k-step each)
  using Lds = PrefillLds<DK, DV>;
  constexpr int KS = Lds::KS, VS = Lds::VS, MS = Lds::MS, TB = Lds::TB;
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
  constexpr int EB = BF ? 2 : 4;  // bytes per base element
  const auto brsrc = make_rsrc(static_cast<const char*>(pa.base) + static_cast<size_t>(tile) * DK * DV * EB,
                               DK * DV * EB);
  const uint32_t bvoff = static_cast<uint32_t>((4 * lg * DV + col0 + ln) * EB);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[kb][cb][r] = ld_base<BF>(brsrc, bvoff, ((16 * kb + r) * DV + 16 * cb) * EB);

  const bool kla = a.eta != nullptr;
  // Inputs of the next chunk are loaded into registers while this chunk is computed;
  // each job is one 16-byte piece (8 channels) of one token.
  constexpr int KP = DK / 8, VP = DV / 8;                         // pieces per row
  constexpr int NPK = C * KP, NPV = C * VP;                       // (token, piece) jobs
  constexpr int LK = (NPK + NT - 1) / NT, LV = (NPV + NT - 1) / NT;
  uint4 nk[LK], nq[LK], nv[LV];
  float ndec = 1.f, nbt = 0.f;
  auto rows_of = [&](const void* x, int t0, int bytes_per_row) { return chunk_rows(x, bseq, h, T, H, t0, bytes_per_row); };
  auto fetch = [&](int t0) {
    const auto rk = rows_of(a.k, t0, 2 * DK), rq = rows_of(a.q, t0, 2 * DK), rv = rows_of(a.v, t0, 2 * DV);
#pragma unroll
    for (int i = 0; i < LK; ++i) {
      const int pc = tid + i * NT, tok = pc / KP, seg = pc % KP;  // jobs past the chunk read zeros
      const uint32_t off = static_cast<uint32_t>((tok * H * DK + seg * 8) * 2);
      nk[i] = bload16(rk, off);
      nq[i] = bload16(rq, off);
    }
#pragma unroll
    for (int i = 0; i < LV; ++i) {
      const int pc = tid + i * NT, tok = pc / VP, seg = pc % VP;
      nv[i] = bload16(rv, static_cast<uint32_t>((tok * H * DV + seg * 8) * 2));
    }
    if (wave == 3) {  // lanes past the chunk or the prompt read zeros
      const uint32_t off = static_cast<uint32_t>(lane * H * 4);
      ndec = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rows_of(a.decay, t0, 4), off, 0, 0));
      nbt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rows_of(kla ? a.eta : a.beta, t0, 4), off, 0, 0));
    }
  };
  fetch(0);
  for (int e = tid; e < 16 * TB; e += NT) {  // rows 0..15 (tokens 16..31 stay zero)
    sh.t1h[e] = 0;
    sh.t1l[e] = 0;
  }

  for (int t0 = 0; t0 < T; t0 += C) {
    __syncthreads();  // every wave is done with the previous chunk's LDS arrays

    // ---- 1. this chunk's rows of K, Q, V (zeros past the end) into LDS; ||k||^2; decays
#pragma unroll
    for (int i = 0; i < LK; ++i) {
      const int pc = tid + i * NT, tok = pc / KP, seg = pc % KP;
      if (pc < NPK) {
        st_kperm8(&sh.k[tok * KS], seg * 8, nk[i]);
        st_kperm8(&sh.q[tok * KS], seg * 8, nq[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < LV; ++i) {
      const int pc = tid + i * NT, tok = pc / VP, seg = pc % VP;
      if (pc < NPV) *reinterpret_cast<uint4*>(&sh.v[tok * VS + seg * 8]) = nv[i];
    }
    if (wave == 3) {
      // lanes 0..31: one token each; inclusive prefix sum of the clamped log2 decays
      const float l2 = scan32((lane < C && t0 + lane < T) ? chunk_log2_decay(ndec) : 0.f);
      if (lane < C) {
        sh.c[lane] = l2;
        sh.gam[lane] = fexp2(l2);
        sh.braw[lane] = nbt;
      }
    }
    if (t0 + C < T) fetch(t0 + C);
    __syncthreads();

    // ---- 2. G = K K^T and P = Q K^T on the lower blocks (six blocks over the first waves);
    //         the step sizes, from G's diagonal for the Kaczmarz one
    constexpr int BPW = NWV >= 6 ? 1 : 2;  // blocks per wave
    if (wave < 6 / BPW) {
#pragma unroll
      for (int e = 0; e < BPW; ++e) {
        const int blk = BPW * wave + e;  // 0..2: G blocks (0,0), (1,0), (1,1); 3..5: the same of P
        const int sub = blk % 3;
        const int ib = sub == 0 ? 0 : 1, jb = sub == 2 ? 1 : 0;
        const uint16_t* xa = blk < 3 ? sh.k : sh.q;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk)  // both operands in the same (storage) channel order
          acc = mma(ld_b128(&xa[(16 * ib + ln) * KS + 32 * kk + 8 * lg]),
                    ld_b128(&sh.k[(16 * jb + ln) * KS + 32 * kk + 8 * lg]), acc);
        float* dst = blk < 3 ? sh.g : sh.p;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * ib + 4 * lg + r) * MS + 16 * jb + ln] = acc[r];
        if ((blk == 0 || blk == 2) && lg == (ln >> 2)) {  // G's diagonal entry (ln, ln): ||k||^2
          const int i = 16 * ib + ln, r = ln & 3;
          const float kk = r == 0 ? acc[0] : r == 1 ? acc[1] : r == 2 ? acc[2] : acc[3];
          sh.beta[i] = t0 + i >= T ? 0.f : kla ? sh.braw[i] / (kk + a.eps) : sh.braw[i];
        }
      }
    }
    __syncthreads();

    // ---- 3. A = strictly lower b_i 2^(c_i - c_j) G_ij (in place); M o P split.  Thread:
    //         columns j, j + 1 (adjacent in k order too) of rows i, i + NT / 16, ...
    {
      constexpr int RPT = C * C / (2 * NT);  // rows a thread
      const int j = 2 * (tid % 16);
      const float cj0 = sh.c[j], cj1 = sh.c[j + 1];
#pragma unroll
      for (int e = 0; e < RPT; ++e) {
        const int i = tid / 16 + (NT / 16) * e;
        const float ci = sh.c[i], bi = sh.beta[i];
        const float d0 = fexp2(fminf(ci - cj0, 0.f)), d1 = fexp2(fminf(ci - cj1, 0.f));  // used where j <= i
        float2 gv = *reinterpret_cast<const float2*>(&sh.g[i * MS + j]);
        const float2 pv = *reinterpret_cast<const float2*>(&sh.p[i * MS + j]);
        if (j < i) gv.x *= bi * d0;
        if (j + 1 < i) gv.y *= bi * d1;
        *reinterpret_cast<float2*>(&sh.g[i * MS + j]) = gv;
        uint32_t hi, lo;
        split2(j <= i ? d0 * pv.x : 0.f, j + 1 <= i ? d1 * pv.y : 0.f, hi, lo);
        *reinterpret_cast<uint32_t*>(&sh.pmh[i * TB + kperm(j)]) = hi;
        *reinterpret_cast<uint32_t*>(&sh.pml[i * TB + kperm(j)]) = lo;
      }
    }
    __syncthreads();

    // ---- 4, 5, 6. T = (I + A)^-1 (T aliasing P from here on); T diag(b), split, in k
    //               order (the A operand of T diag(b) R below)
    invert_unit_lower32<MS, TB, NT>(sh.g, sh.t, sh.xs, sh.beta, sh.t1h, sh.t1l, tid);

    // ---- 7, 8. X = K S and Q S (S split one channel-block pair at a time; K and Q are
    //            exact bf16 operands); R = V - diag(g) X in fp32 at X's accumulator
    //            positions (tokens 4 lg + r and 16 + 4 lg + r), which makes R the B operand
    //            of U = T diag(b) R with the tokens paired the same way in the A operand;
    //            and (diag(g) Q S)^T for the outputs (S as the A operand: lanes hold tokens)
    //            S is replaced by g_C S (the first term of the update in step 10) as it is
    //            split, so the split's remainders are formed in the old S's registers
    float U[2][NCB][4], O[2][NCB][4];
    const float gC = sh.gam[C - 1], cC = sh.c[C - 1];
    {
      f32x4 xs[2][NCB], qs[2][NCB];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          xs[ib][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
          qs[ib][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int kp = 0; kp < NKP; ++kp) {
        bf16x8 shi[NCB], slo[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          float x0[4], x1[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x0[r] = S[2 * kp][cb][r];
            x1[r] = S[2 * kp + 1][cb][r];
            S[2 * kp][cb][r] = gC * x0[r];
            S[2 * kp + 1][cb][r] = gC * x1[r];
          }
          split_pair(x0, x1, shi[cb], slo[cb]);
        }
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
          const int rowk = (16 * ib + ln) * KS + 32 * kp + 8 * lg;  // channels 32 kp + 4 lg + {0..3, 16..19}
          const bf16x8 ka = ld_b128(&sh.k[rowk]);
          const bf16x8 qa = ld_b128(&sh.q[rowk]);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            xs[ib][cb] = mma(ka, shi[cb], xs[ib][cb]);
            xs[ib][cb] = mma(ka, slo[cb], xs[ib][cb]);
            qs[ib][cb] = mma(shi[cb], qa, qs[ib][cb]);
            qs[ib][cb] = mma(slo[cb], qa, qs[ib][cb]);
          }
        }
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        float vf[8];  // V at this lane's accumulator positions
        unpack8(__builtin_bit_cast(uint4, ld_tr8(sh.v, VS, 4 * lg, 16 + 4 * lg, col0 + 16 * cb, ln)), vf);
        float r0[4], r1[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          r0[r] = fmaf(-sh.gam[4 * lg + r], xs[0][cb][r], vf[r]);
          r1[r] = fmaf(-sh.gam[16 + 4 * lg + r], xs[1][cb][r], vf[4 + r]);
        }
        bf16x8 rhi, rlo;
        split_pair(r0, r1, rhi, rlo);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
          const int rowt = (16 * ib + ln) * TB + 8 * lg;
          const bf16x8 tah = ld_b128(&sh.t1h[rowt]);
          const bf16x8 tal = ld_b128(&sh.t1l[rowt]);
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          acc = mma(tah, rhi, acc);
          acc = mma(tah, rlo, acc);
          acc = mma(tal, rhi, acc);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            U[ib][cb][r] = acc[r];
            O[ib][cb][r] = sh.gam[16 * ib + ln] * qs[ib][cb][r];
          }
        }
      }
    }

    // ---- 9. O^T += U^T (M o Q K^T)^T; write the outputs (lane: token 16 ib + ln,
    //         columns 16 cb + 4 lg .. + 3).  diag(2^(c_C - c_j)) U, the factor of the
    //         update in step 10, is formed first, so the split below consumes U.
    float U2[2][NCB][4];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float f = fexp2(cC - sh.c[16 * ib + 4 * lg + r]);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) U2[ib][cb][r] = U[ib][cb][r] * f;
      }
    const auto orows = out_rows(a.out, bseq, T, H, DV, t0, C);
    const uint32_t olane = static_cast<uint32_t>((ln * H + static_cast<int>(h)) * DV + col0 + 4 * lg) * 4;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      bf16x8 uhi, ulo;
      split_pair(U[0][cb], U[1][cb], uhi, ulo);
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        const int rowp = (16 * ib + ln) * TB + 8 * lg;
        const bf16x8 pah = ld_b128(&sh.pmh[rowp]);
        const bf16x8 pal = ld_b128(&sh.pml[rowp]);
        f32x4 acc = {O[ib][cb][0], O[ib][cb][1], O[ib][cb][2], O[ib][cb][3]};
        acc = mma(uhi, pah, acc);
        acc = mma(ulo, pah, acc);
        acc = mma(uhi, pal, acc);
        st_out4(orows, olane + static_cast<uint32_t>(16 * ib * H * DV + 16 * cb) * 4, acc);
      }
    }

    // ---- 10. S = g_C S + K^T (diag(2^(c_C - c_j)) U), g_C S formed in step 7
    bf16x8 u2hi[NCB], u2lo[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) split_pair(U2[0][cb], U2[1][cb], u2hi[cb], u2lo[cb]);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      // K^T, tokens as U's rows; this lane's 4 channels 16 kb + 4 (ln % 4) in storage order
      const bf16x8 ka = ld_tr8_at(sh.k, KS, 4 * lg, 16 + 4 * lg, kperm(16 * kb + 4 * (ln & 3)), ln);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        f32x4 acc = {S[kb][cb][0], S[kb][cb][1], S[kb][cb][2], S[kb][cb][3]};
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
      for (int r = 0; r < 4; ++r) st_base<BF>(brsrc, bvoff, ((16 * kb + r) * DV + 16 * cb) * EB, S[kb][cb][r]);
}



// In-place prefix sums over the 32 tokens of a chunk, for each of DK channels of a
// [token][channel] fp32 array with row stride CS: thread (channel, half) adds up 16
// tokens in registers and the second half adds the first half's total.  glast[ch]
// receives 2 to the power of the last token's sum.
template <int DK, int CS>
__device__ __forceinline__ void prefix_over_tokens(float* cc, float* glast, int tid) {
  const int ch = tid >> 1, hf = tid & 1;
  if (ch < DK) {  // whole waves
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = cc[(16 * hf + i) * CS + ch];
#pragma unroll
    for (int i = 1; i < 16; ++i) x[i] += x[i - 1];
    const float first = __shfl_xor(x[15], 1, 64);  // the partner's total
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (hf == 1) x[i] += first;
      cc[(16 * hf + i) * CS + ch] = x[i];
    }
    if (hf == 1) glast[ch] = fexp2(x[15]);  // 2^c of the chunk's last token
  }
}

// ------------------------------------------------------------------ KDA prefill
// KDA decays each key channel on its own: with G_i = a_1 ... a_i (a dk-vector,
// cumulative within the chunk, kept as log2 in cc) the chunk form becomes
//   A_ij = b_i sum_c k_i[c] k_j[c] G_i[c] / G_j[c]  (j < i),   T = (I + A)^-1
//   U    = T diag(b) (V - (K o G) S)
//   O    = (Q o G) S + P U,   P_ij = sum_c q_i[c] k_j[c] G_i[c] / G_j[c]  (j <= i)
//   S'   = diag(G_C) S + (K o G_C / G)^T U
// (the same unrolling of u_i as for GDN, with diag(G) in place of the scalar g).
// Every product runs on MFMA with the decay folded into a split operand; the
// decay-weighted C x C products A and P use a reference token per block (step 4) and
// fall back to forming each pair directly when a chunk's decays are too strong for it.
template <int DK, int DV>
struct PrefillKdaLds {
  static constexpr int C = kChunk;
  // Row strides (bf16) of 8 mod 16 words, for 16-byte and transposing reads (see PrefillLds).
  static constexpr int KS = DK + 16;  // K, Q, K o G and Q o G (the last two in k order, kperm)
  static constexpr int RS = DK + 16;  // bf16 row stride of K o G_C / G, and
  static constexpr int VS = DV + 16;  // of V: 8 mod 32 words (transposing reads)
  static constexpr int MS = C + 4;    // fp32 row stride of the C x C matrices (16-byte rows)
  static constexpr int TB = C + 16;  // split C x C matrices
  static constexpr int CS = DK + 8;  // fp32 row stride of the per-channel decays
  float beta[C];
  float braw[C];
  float knorm[C];
  float glast[DK];  // 2^c of the chunk's last token per channel
  float g[C * MS];  // A (strictly lower part)
  float t[C * MS];    // the diagonal blocks of T = (I + A)^-1
  float xs[16 * 17];  // scratch of the inverse
  uint16_t t1h[C * TB];  // T diag(b) (hi part, k order; upper right block zero)
  uint16_t t1l[C * TB];
  uint16_t pmh[C * TB], pml[C * TB];  // P (lower triangle, split, k order)
  uint16_t k[C * KS];  // K, token rows
  uint16_t q[C * KS];  // Q, token rows
  uint16_t qgh[C * KS], qgl[C * KS];  // Q o G, token rows, split, k order
  uint16_t v[C * VS];                 // V, token rows
  float part[4 * 6 * 4 * 64];         // per-wave partial sums of A and P
  uint16_t kgh[C * KS], kgl[C * KS];  // K o G, token rows, split, k order
  uint16_t kdh[C * RS], kdl[C * RS];  // K o G_C / G, token rows, split
  float cc[C * CS];                   // log2 decays, then their prefix sums over the chunk
};

// KDA workgroup size: 8 waves, 16 value columns each, when dv = 128 (two waves share each
// SIMD, since the LDS of one tile leaves room for one workgroup per CU), else 4.
template <int DV>
constexpr int kda_threads() { return DV == 128 ? 512 : 256; }

template <int DK, int DV, bool BF>
__global__ void __launch_bounds__(kda_threads<DV>()) prefill_kda_kernel(PoolArgs pa, PrefillArgs a) {
  constexpr int C = kChunk;
  constexpr int NT = kda_threads<DV>(), NWV = NT / 64;  // threads, waves
  constexpr int CW = DV / NWV;
  constexpr int NCB = CW / 16;
  constexpr int NKB = DK / 16;
  constexpr int NKP = DK / 32;
  using Lds = PrefillKdaLds<DK, DV>;
  constexpr int KS = Lds::KS, RS = Lds::RS, VS = Lds::VS, MS = Lds::MS, TB = Lds::TB;
  constexpr int CS = Lds::CS;
  __shared__ __align__(16) Lds sh;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int tile = blockIdx.x;
  const int H = pa.heads, T = a.tokens;
  const size_t bseq = static_cast<size_t>(tile / H), h = static_cast<size_t>(tile % H);
  const int col0 = wave * CW;

  float S[NKB][NCB][4];
  constexpr int EB = BF ? 2 : 4;
  const auto brsrc = make_rsrc(static_cast<const char*>(pa.base) + static_cast<size_t>(tile) * DK * DV * EB,
                               DK * DV * EB);
  const uint32_t bvoff = static_cast<uint32_t>((4 * lg * DV + col0 + ln) * EB);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[kb][cb][r] = ld_base<BF>(brsrc, bvoff, ((16 * kb + r) * DV + 16 * cb) * EB);

  const bool kla = a.eta != nullptr;
  constexpr int KP = DK / 8, VP = DV / 8;
  constexpr int NPK = C * KP, NPV = C * VP;  // (token, piece) jobs
  constexpr int LK = (NPK + NT - 1) / NT, LV = (NPV + NT - 1) / NT;
  constexpr int ND = C * DK / 4 / NT;  // float4 decay pieces per thread
  uint4 nk[LK], nq[LK], nv[LV];
  float4 nd[ND];
  float nbt = 0.f;
  auto rows_of = [&](const void* x, int t0, int bytes_per_row) { return chunk_rows(x, bseq, h, T, H, t0, bytes_per_row); };
  auto fetch = [&](int t0) {  // rows past the prompt read as zeros
    const auto rk = rows_of(a.k, t0, 2 * DK), rq = rows_of(a.q, t0, 2 * DK), rv = rows_of(a.v, t0, 2 * DV);
    const auto rd = rows_of(a.decay, t0, 4 * DK);
#pragma unroll
    for (int i = 0; i < LK; ++i) {
      const int pc = tid + i * NT, tok = pc / KP, seg = pc % KP;  // jobs past the chunk read zeros
      const uint32_t off = static_cast<uint32_t>((tok * H * DK + seg * 8) * 2);
      nk[i] = bload16(rk, off);
      nq[i] = bload16(rq, off);
    }
#pragma unroll
    for (int i = 0; i < LV; ++i) {
      const int pc = tid + i * NT, tok = pc / VP, seg = pc % VP;
      nv[i] = bload16(rv, static_cast<uint32_t>((tok * H * DV + seg * 8) * 2));
    }
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const int pc = tid + i * NT, tok = pc / (DK / 4), seg = pc % (DK / 4);
      const uint4 w = bload16(rd, static_cast<uint32_t>((tok * H * DK + seg * 4) * 4));
      nd[i] = make_float4(__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w));
    }
    if (wave == 3)
      nbt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rows_of(kla ? a.eta : a.beta, t0, 4),
                                                                 static_cast<uint32_t>(lane * H * 4), 0, 0));
  };
  fetch(0);
  // entries above the diagonal of P and the upper right block of the split T: written once
  for (int e = tid; e < C * C; e += NT) {
    const int i = e / C, j = e % C;
    if (j > i) {
      sh.pmh[i * TB + kperm(j)] = 0;
      sh.pml[i * TB + kperm(j)] = 0;
    }
    if (i < 16 && j >= 16) {
      sh.t1h[i * TB + kperm(j)] = 0;
      sh.t1l[i * TB + kperm(j)] = 0;
    }
  }

  for (int t0 = 0; t0 < T; t0 += C) {
    __syncthreads();

    // ---- 1. K, Q and V rows; clamped log2 decays; ||k||^2; step sizes
#pragma unroll
    for (int i = 0; i < LK; ++i) {
      const int pc = tid + i * NT, tok = pc / KP, seg = pc % KP;
      if (pc < NPK) {
        *reinterpret_cast<uint4*>(&sh.k[tok * KS + seg * 8]) = nk[i];
        *reinterpret_cast<uint4*>(&sh.q[tok * KS + seg * 8]) = nq[i];
        if (kla) {
          float f[8];
          unpack8(nk[i], f);
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
          ss = group_sum<KP>(ss);
          if (seg == 0) sh.knorm[tok] = ss;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < LV; ++i) {
      const int pc = tid + i * NT, tok = pc / VP, seg = pc % VP;
      if (pc < NPV) *reinterpret_cast<uint4*>(&sh.v[tok * VS + seg * 8]) = nv[i];
    }
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const int pc = tid + i * NT, tok = pc / (DK / 4), seg = pc % (DK / 4);
      const bool ok = t0 + tok < T;  // tokens past the prompt do not decay the state
      *reinterpret_cast<float4*>(&sh.cc[tok * CS + seg * 4]) =
          make_float4(ok ? chunk_log2_decay(nd[i].x) : 0.f, ok ? chunk_log2_decay(nd[i].y) : 0.f,
                      ok ? chunk_log2_decay(nd[i].z) : 0.f, ok ? chunk_log2_decay(nd[i].w) : 0.f);
    }
    if (wave == 3 && lane < C) sh.braw[lane] = nbt;
    if (t0 + C < T) fetch(t0 + C);
    __syncthreads();

    // ---- 2. prefix sums of the log2 decays over the chunk's tokens; step sizes
    prefix_over_tokens<DK, CS>(sh.cc, sh.glast, tid);
    if (tid < C) {
      const bool ok = t0 + tid < T;
      sh.beta[tid] = !ok ? 0.f : kla ? sh.braw[tid] / (sh.knorm[tid] + a.eps) : sh.braw[tid];
    }
    __syncthreads();

    // ---- 3. decay-folded operands Q o G, K o G and K o G_C / G (token rows), split;
    //         thread (token, 8-channel segment)
    for (int pc = tid; pc < C * KP; pc += NT) {
      const int tok = pc / KP, seg = pc % KP;
      float kf[8], qf[8], cf[8], cl[8];
      unpack8(*reinterpret_cast<const uint4*>(&sh.k[tok * KS + seg * 8]), kf);
      unpack8(*reinterpret_cast<const uint4*>(&sh.q[tok * KS + seg * 8]), qf);
      load8(&sh.cc[tok * CS + seg * 8], cf);
      load8(&sh.cc[(C - 1) * CS + seg * 8], cl);
      uint32_t qh[4], ql[4], kgh2[4], kgl2[4], kdh2[4], kdl2[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {  // channels e, e + 1 packed
        const float g0 = fexp2(cf[e]), g1 = fexp2(cf[e + 1]);
        split2(qf[e] * g0, qf[e + 1] * g1, qh[e / 2], ql[e / 2]);
        split2(kf[e] * g0, kf[e + 1] * g1, kgh2[e / 2], kgl2[e / 2]);
        split2(kf[e] * fexp2(cl[e] - cf[e]), kf[e + 1] * fexp2(cl[e + 1] - cf[e + 1]), kdh2[e / 2], kdl2[e / 2]);
      }
      st_kperm8(&sh.qgh[tok * KS], seg * 8, make_uint4(qh[0], qh[1], qh[2], qh[3]));
      st_kperm8(&sh.qgl[tok * KS], seg * 8, make_uint4(ql[0], ql[1], ql[2], ql[3]));
      st_kperm8(&sh.kgh[tok * KS], seg * 8, make_uint4(kgh2[0], kgh2[1], kgh2[2], kgh2[3]));
      st_kperm8(&sh.kgl[tok * KS], seg * 8, make_uint4(kgl2[0], kgl2[1], kgl2[2], kgl2[3]));
      *reinterpret_cast<uint4*>(&sh.kdh[tok * RS + seg * 8]) = make_uint4(kdh2[0], kdh2[1], kdh2[2], kdh2[3]);
      *reinterpret_cast<uint4*>(&sh.kdl[tok * RS + seg * 8]) = make_uint4(kdl2[0], kdl2[1], kdl2[2], kdl2[3]);
    }

    // ---- 4. A and P.  G_i / G_j = (G_i / G_R)(G_R / G_j) splits the decay of a pair
    //        around a reference token R: R = start of the chunk for the block of
    //        rows and columns 0..15, R = token 15 for the blocks of rows 16..31.
    //        Row factors are then <= 1 and column factors at most the decay over 16
    //        tokens, so when no channel decays by more than 2^-60 over either half of
    //        the chunk the products run on MFMA with three-way split operands (these
    //        sums over channels can cancel, so they keep 24 bits).  Each wave takes 32
    //        channels of A and P (with eight waves, of block (0,0) or of the two blocks
    //        of rows 16..31; with four, of all three), building each row and column
    //        operand once; the partial sums over channel steps are added in a fixed
    //        order through LDS.
    //        Otherwise every pair is formed directly.
    bool direct;
    {
      bool big = false;
      for (int ch = tid; ch < DK; ch += NT)
        big = big || -sh.cc[15 * CS + ch] > 60.f || sh.cc[15 * CS + ch] - sh.cc[(C - 1) * CS + ch] > 60.f;
      direct = __syncthreads_or(big);
    }
    if (!direct) {
      constexpr int NKS = DK / 32;   // 32-channel steps
      constexpr int SPLIT = NWV / 4;  // 2: waves 0..3 take block (0,0), waves 4..7 the blocks
                                      //    (1,0) and (1,1); 1: each wave all three
      const int ks0 = wave & 3;
      const bool top = SPLIT == 1 || wave < 4, bottom = SPLIT == 1 || wave >= 4;
      // acc: A and P of the blocks (0,0), (1,0), (1,1) in that order (A even, P odd)
      f32x4 acc[6];
#pragma unroll
      for (int m = 0; m < 6; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
      auto ops = [](const uint32_t (&w)[3][4], bf16x8 (&x)[3]) {
#pragma unroll
        for (int u = 0; u < 3; ++u) x[u] = pack8(w[u][0], w[u][1], w[u][2], w[u][3]);
      };
      for (int kk = ks0; kk < NKS; kk += 4) {
        const int ch0 = 32 * kk + 8 * lg;
        float ref[8];
        load8(&sh.cc[15 * CS + ch0], ref);
        if (top) {  // rows: token ln with R = start; columns: token ln with R = start
          float c0[8], k0[8], q0[8];
          load8(&sh.cc[ln * CS + ch0], c0);
          unpack8(*reinterpret_cast<const uint4*>(&sh.k[ln * KS + ch0]), k0);
          unpack8(*reinterpret_cast<const uint4*>(&sh.q[ln * KS + ch0]), q0);
          uint32_t ka[3][4], qa[3][4], c00[3][4];
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float r0a = fexp2(c0[e]), r0b = fexp2(c0[e + 1]);
            split3(k0[e] * r0a, k0[e + 1] * r0b, ka[0][e / 2], ka[1][e / 2], ka[2][e / 2]);
            split3(q0[e] * r0a, q0[e + 1] * r0b, qa[0][e / 2], qa[1][e / 2], qa[2][e / 2]);
            split3(k0[e] * fexp2(-c0[e]), k0[e + 1] * fexp2(-c0[e + 1]), c00[0][e / 2], c00[1][e / 2],
                   c00[2][e / 2]);
          }
          bf16x8 KA[3], QA[3], C00[3];
          ops(ka, KA);
          ops(qa, QA);
          ops(c00, C00);
          acc[0] = mma3(KA, C00, acc[0]);
          acc[1] = mma3(QA, C00, acc[1]);
        }
        if (bottom) {  // rows: token 16 + ln with R = 15; columns: token ln and 16 + ln with R = 15
          float c0[8], c1[8], k0[8], k1[8], q1[8];
          load8(&sh.cc[ln * CS + ch0], c0);
          load8(&sh.cc[(16 + ln) * CS + ch0], c1);
          unpack8(*reinterpret_cast<const uint4*>(&sh.k[ln * KS + ch0]), k0);
          unpack8(*reinterpret_cast<const uint4*>(&sh.k[(16 + ln) * KS + ch0]), k1);
          unpack8(*reinterpret_cast<const uint4*>(&sh.q[(16 + ln) * KS + ch0]), q1);
          uint32_t kb[3][4], qb[3][4], c10[3][4], c11[3][4];
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float r1a = fexp2(c1[e] - ref[e]), r1b = fexp2(c1[e + 1] - ref[e + 1]);
            split3(k1[e] * r1a, k1[e + 1] * r1b, kb[0][e / 2], kb[1][e / 2], kb[2][e / 2]);
            split3(q1[e] * r1a, q1[e + 1] * r1b, qb[0][e / 2], qb[1][e / 2], qb[2][e / 2]);
            split3(k0[e] * fexp2(ref[e] - c0[e]), k0[e + 1] * fexp2(ref[e + 1] - c0[e + 1]), c10[0][e / 2],
                   c10[1][e / 2], c10[2][e / 2]);
            split3(k1[e] * fexp2(ref[e] - c1[e]), k1[e + 1] * fexp2(ref[e + 1] - c1[e + 1]), c11[0][e / 2],
                   c11[1][e / 2], c11[2][e / 2]);
          }
          bf16x8 KB[3], QB[3], C10[3], C11[3];
          ops(kb, KB);
          ops(qb, QB);
          ops(c10, C10);
          ops(c11, C11);
          acc[2] = mma3(KB, C10, acc[2]);
          acc[3] = mma3(QB, C10, acc[3]);
          acc[4] = mma3(KB, C11, acc[4]);
          acc[5] = mma3(QB, C11, acc[5]);
        }
      }
      // part[channel step][m][r][lane], each entry written by the one wave that formed it
      constexpr int NKW = NKS < 4 ? NKS : 4;  // channel steps held
      if (ks0 < NKW) {
#pragma unroll
        for (int m = 0; m < 6; ++m) {
          if (m < 2 ? !top : !bottom) continue;
#pragma unroll
          for (int r = 0; r < 4; ++r) sh.part[((ks0 * 6 + m) * 4 + r) * 64 + lane] = acc[m][r];
        }
      }
      __syncthreads();
      // thread (r = wave % 4, lane): entry r of this lane in the block products (with eight
      // waves, waves 0..3 finish A and waves 4..7 P), partial sums added in channel order
      const int r = wave & 3, j0 = ln;
#pragma unroll
      for (int m = 0; m < 6; ++m) {
        if (SPLIT == 2 && (m & 1) != (wave >> 2)) continue;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < NKW; ++w) sum += sh.part[((w * 6 + m) * 4 + r) * 64 + lane];
        const int blk = m >> 1, ib = blk == 0 ? 0 : 1, jb = blk == 2 ? 1 : 0;
        const int i = 16 * ib + 4 * lg + r, j = 16 * jb + j0;
        if ((m & 1) == 0) {
          sh.g[i * MS + j] = j < i ? sh.beta[i] * sum : 0.f;
        } else {
          uint32_t hi, lo;
          split2(j <= i ? sum : 0.f, 0.f, hi, lo);
          sh.pmh[i * TB + kperm(j)] = static_cast<uint16_t>(hi);
          sh.pml[i * TB + kperm(j)] = static_cast<uint16_t>(lo);
        }
      }
    } else if (tid < 256) {
      // pairwise: thread (row pair ip, ip' = 31 - ip; channel slice sl)
      constexpr int SL = DK / 16;  // channels per slice
      const int ip = tid >> 4, sl = tid & 15;
      float kr[2][SL], qr[2][SL], cr[2][SL];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int r = w == 0 ? ip : C - 1 - ip;
#pragma unroll
        for (int e = 0; e < SL; ++e) {
          kr[w][e] = bf16_to_f32(sh.k[r * KS + sl * SL + e]);
          qr[w][e] = bf16_to_f32(sh.q[r * KS + sl * SL + e]);
          cr[w][e] = sh.cc[r * CS + sl * SL + e];
        }
      }
      for (int n = 0; n <= C; ++n) {  // row ip takes j = 0..ip, row 31 - ip takes j = 0..31 - ip
        const bool first = n <= ip;
        const int r = first ? ip : C - 1 - ip, j = first ? n : n - ip - 1;
        float av = 0.f, pv = 0.f;
#pragma unroll
        for (int e = 0; e < SL; ++e) {
          const float u = bf16_to_f32(sh.k[j * KS + sl * SL + e]) *
                          fexp2((first ? cr[0][e] : cr[1][e]) - sh.cc[j * CS + sl * SL + e]);
          av = fmaf(first ? kr[0][e] : kr[1][e], u, av);
          pv = fmaf(first ? qr[0][e] : qr[1][e], u, pv);
        }
        av = group_sum<16>(av);
        pv = group_sum<16>(pv);
        if (sl == 0) {
          if (j < r) sh.g[r * MS + j] = sh.beta[r] * av;
          uint32_t hi, lo;
          split2(pv, 0.f, hi, lo);
          sh.pmh[r * TB + kperm(j)] = static_cast<uint16_t>(hi);
          sh.pml[r * TB + kperm(j)] = static_cast<uint16_t>(lo);
        }
      }
    }
    __syncthreads();

    // ---- 5, 6. T = (I + A)^-1; T diag(b), split, in k order (the A operand of
    //            T diag(b) R below)
    invert_unit_lower32<MS, TB, NT>(sh.g, sh.t, sh.xs, sh.beta, sh.t1h, sh.t1l, tid);

    // ---- 7, 8. X = (K o G) S and ((Q o G) S)^T (split operands, S one channel-block pair
    //            at a time; S is the A operand of the second, so its lanes hold tokens);
    //            R = V - X in fp32 at X's accumulator positions, the B operand of
    //            U = T diag(b) R.  S is replaced by diag(G_C) S (the first term of the
    //            update in step 10) as it is split, so the split consumes the old S.
    float U[2][NCB][4], O[2][NCB][4];
    {
      f32x4 xs[2][NCB], qs[2][NCB];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          xs[ib][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
          qs[ib][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int kp = 0; kp < NKP; ++kp) {
        bf16x8 shi[NCB], slo[NCB];
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(&sh.glast[32 * kp + 4 * lg]);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(&sh.glast[32 * kp + 16 + 4 * lg]);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          float x0[4], x1[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x0[r] = S[2 * kp][cb][r];
            x1[r] = S[2 * kp + 1][cb][r];
            S[2 * kp][cb][r] = g0[r] * x0[r];
            S[2 * kp + 1][cb][r] = g1[r] * x1[r];
          }
          split_pair(x0, x1, shi[cb], slo[cb]);
        }
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
          const int rowk = (16 * ib + ln) * KS + 32 * kp + 8 * lg;  // channels 32 kp + 4 lg + {0..3, 16..19}
          const bf16x8 kah = ld_b128(&sh.kgh[rowk]), kal = ld_b128(&sh.kgl[rowk]);
          const bf16x8 qah = ld_b128(&sh.qgh[rowk]), qal = ld_b128(&sh.qgl[rowk]);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            xs[ib][cb] = mma(kah, shi[cb], xs[ib][cb]);
            xs[ib][cb] = mma(kah, slo[cb], xs[ib][cb]);
            xs[ib][cb] = mma(kal, shi[cb], xs[ib][cb]);
            qs[ib][cb] = mma(shi[cb], qah, qs[ib][cb]);
            qs[ib][cb] = mma(slo[cb], qah, qs[ib][cb]);
            qs[ib][cb] = mma(shi[cb], qal, qs[ib][cb]);
          }
        }
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        float vf[8];  // V at this lane's accumulator positions
        unpack8(__builtin_bit_cast(uint4, ld_tr8(sh.v, VS, 4 * lg, 16 + 4 * lg, col0 + 16 * cb, ln)), vf);
        float r0[4], r1[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          r0[r] = vf[r] - xs[0][cb][r];
          r1[r] = vf[4 + r] - xs[1][cb][r];
        }
        bf16x8 rhi, rlo;
        split_pair(r0, r1, rhi, rlo);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
          const int rowt = (16 * ib + ln) * TB + 8 * lg;
          const bf16x8 tah = ld_b128(&sh.t1h[rowt]);
          const bf16x8 tal = ld_b128(&sh.t1l[rowt]);
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          acc = mma(tah, rhi, acc);
          acc = mma(tah, rlo, acc);
          acc = mma(tal, rhi, acc);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            U[ib][cb][r] = acc[r];
            O[ib][cb][r] = qs[ib][cb][r];
          }
        }
      }
    }

    // ---- 9. O^T += U^T P^T; outputs (lane: token 16 ib + ln, columns 16 cb + 4 lg .. + 3).
    //         U's split serves here and in step 10.
    bf16x8 uhi[NCB], ulo[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) split_pair(U[0][cb], U[1][cb], uhi[cb], ulo[cb]);
    const auto orows = out_rows(a.out, bseq, T, H, DV, t0, C);
    const uint32_t olane = static_cast<uint32_t>((ln * H + static_cast<int>(h)) * DV + col0 + 4 * lg) * 4;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        const int rowp = (16 * ib + ln) * TB + 8 * lg;
        const bf16x8 pah = ld_b128(&sh.pmh[rowp]), pal = ld_b128(&sh.pml[rowp]);
        f32x4 acc = {O[ib][cb][0], O[ib][cb][1], O[ib][cb][2], O[ib][cb][3]};
        acc = mma(uhi[cb], pah, acc);
        acc = mma(ulo[cb], pah, acc);
        acc = mma(uhi[cb], pal, acc);
        st_out4(orows, olane + static_cast<uint32_t>(16 * ib * H * DV + 16 * cb) * 4, acc);
      }
    }

    // ---- 10. S = diag(G_C) S + (K o G_C / G)^T U, diag(G_C) S formed in step 7
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const bf16x8 kah = ld_tr8(sh.kdh, RS, 4 * lg, 16 + 4 * lg, 16 * kb, ln);  // tokens as U's rows
      const bf16x8 kal = ld_tr8(sh.kdl, RS, 4 * lg, 16 + 4 * lg, 16 * kb, ln);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        f32x4 acc = {S[kb][cb][0], S[kb][cb][1], S[kb][cb][2], S[kb][cb][3]};
        acc = mma(kah, uhi[cb], acc);
        acc = mma(kah, ulo[cb], acc);
        acc = mma(kal, uhi[cb], acc);
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
      for (int r = 0; r < 4; ++r) st_base<BF>(brsrc, bvoff, ((16 * kb + r) * DV + 16 * cb) * EB, S[kb][cb][r]);
}


// ---------------------------------------------------------------- RWKV6 prefill
// RWKV6 reads the state before each token's write and adds a bonus term:
//   o_i = S_{i-1}^T r_i + (sum_c r_i[c] u[c] k_i[c]) v_i,   S_i = diag(w_i) S_{i-1} + k_i v_i^T.
// With G_i = w_1 ... w_i within the chunk (G_-1 = 1; log2 in cc):
//   O  = (R o G_prev) S + P V,   P_ij = sum_c r_i[c] k_j[c] G_{i-1}[c] / G_j[c]  (j < i),
//                                P_ii = sum_c r_i[c] u[c] k_i[c]
//   S' = diag(G_C) S + (K o G_C / G)^T V
// There is no delta-rule solve; V enters every product as an exact bf16 operand.
// P's decay-weighted part uses the same reference-token split (and pairwise
// fallback) as KDA, with the row decay taken one token earlier.
template <int DK, int DV>
struct PrefillRwkvLds {
  static constexpr int C = kChunk;
  static constexpr int KS = DK + 16;  // K, R and R o G_prev rows (the last in k order, kperm)
  static constexpr int RS = DK + 16;  // K o G_C / G and V: 8 mod 16 words (transposing reads)
  static constexpr int VS = DV + 16;
  static constexpr int TB = C + 16;   // P, split (16-byte reads)
  static constexpr int CS = DK + 8;
  float bonus[DK];
  float glast[DK];                    // 2^c of the chunk's last token per channel
  float pd[C];                        // the bonus diagonal of P
  uint16_t pmh[C * TB], pml[C * TB];  // P, split
  uint16_t k[C * KS];                // K, token rows
  uint16_t q[C * KS];                // R, token rows
  uint16_t rgh[C * KS], rgl[C * KS];  // R o G_prev, token rows, split, k order
  uint16_t v[C * VS];                 // V, token rows
  uint16_t kdh[C * RS], kdl[C * RS];  // K o G_C / G, token rows, split
  union {
    float cc[C * CS];              // log2 decays, then their prefix sums
    float part[2 * 3 * 4 * 64];    // after the last read of cc: per-wave partial sums of P
  };
};

// 64 x 64 tiles fit three workgroups per CU (52 KB of LDS, at most 168 VGPRs).
template <int DK, int DV, bool BF>
__global__ void __launch_bounds__(kThreads, DK == 64 && DV == 64 ? 3 : 1) prefill_rwkv_kernel(PoolArgs pa, PrefillArgs a) {
  constexpr int C = kChunk;
  constexpr int CW = DV / 4;
  constexpr int NCB = CW / 16;
  constexpr int NKB = DK / 16;
  constexpr int NKP = DK / 32;
  using Lds = PrefillRwkvLds<DK, DV>;
  constexpr int KS = Lds::KS, RS = Lds::RS, VS = Lds::VS, TB = Lds::TB, CS = Lds::CS;
  __shared__ __align__(16) Lds sh;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int tile = blockIdx.x;
  const int H = pa.heads, T = a.tokens;
  const size_t bseq = static_cast<size_t>(tile / H), h = static_cast<size_t>(tile % H);
  const int col0 = wave * CW;

  float S[NKB][NCB][4];
  constexpr int EB = BF ? 2 : 4;
  const auto brsrc = make_rsrc(static_cast<const char*>(pa.base) + static_cast<size_t>(tile) * DK * DV * EB,
                               DK * DV * EB);
  const uint32_t bvoff = static_cast<uint32_t>((4 * lg * DV + col0 + ln) * EB);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[kb][cb][r] = ld_base<BF>(brsrc, bvoff, ((16 * kb + r) * DV + 16 * cb) * EB);
  for (int ch = tid; ch < DK; ch += kThreads) sh.bonus[ch] = a.bonus[h * DK + ch];

  constexpr int KP = DK / 8, VP = DV / 8;
  constexpr int NPK = C * KP, NPV = C * VP;  // (token, piece) jobs
  constexpr int LK = (NPK + kThreads - 1) / kThreads, LV = (NPV + kThreads - 1) / kThreads;
  constexpr int ND = C * DK / 4 / kThreads;
  uint4 nk[LK], nq[LK], nv[LV];
  float4 nd[ND];
  auto rows_of = [&](const void* x, int t0, int bytes_per_row) { return chunk_rows(x, bseq, h, T, H, t0, bytes_per_row); };
  auto fetch = [&](int t0) {  // rows past the prompt read as zeros
    const auto rk = rows_of(a.k, t0, 2 * DK), rq = rows_of(a.q, t0, 2 * DK), rv = rows_of(a.v, t0, 2 * DV);
    const auto rd = rows_of(a.decay, t0, 4 * DK);
#pragma unroll
    for (int i = 0; i < LK; ++i) {
      const int pc = tid + i * kThreads, tok = pc / KP, seg = pc % KP;  // jobs past the chunk read zeros
      const uint32_t off = static_cast<uint32_t>((tok * H * DK + seg * 8) * 2);
      nk[i] = bload16(rk, off);
      nq[i] = bload16(rq, off);
    }
#pragma unroll
    for (int i = 0; i < LV; ++i) {
      const int pc = tid + i * kThreads, tok = pc / VP, seg = pc % VP;
      nv[i] = bload16(rv, static_cast<uint32_t>((tok * H * DV + seg * 8) * 2));
    }
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const int pc = tid + i * kThreads, tok = pc / (DK / 4), seg = pc % (DK / 4);
      const uint4 w = bload16(rd, static_cast<uint32_t>((tok * H * DK + seg * 4) * 4));
      nd[i] = make_float4(__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w));
    }
  };
  fetch(0);

  for (int t0 = 0; t0 < T; t0 += C) {
    __syncthreads();

    // ---- 1. K, R and V rows; clamped log2 decays
#pragma unroll
    for (int i = 0; i < LK; ++i) {
      const int pc = tid + i * kThreads, tok = pc / KP, seg = pc % KP;
      if (pc < NPK) {
        *reinterpret_cast<uint4*>(&sh.k[tok * KS + seg * 8]) = nk[i];
        *reinterpret_cast<uint4*>(&sh.q[tok * KS + seg * 8]) = nq[i];
      }
    }
#pragma unroll
    for (int i = 0; i < LV; ++i) {
      const int pc = tid + i * kThreads, tok = pc / VP, seg = pc % VP;
      if (pc < NPV) *reinterpret_cast<uint4*>(&sh.v[tok * VS + seg * 8]) = nv[i];
    }
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const int pc = tid + i * kThreads, tok = pc / (DK / 4), seg = pc % (DK / 4);
      const bool ok = t0 + tok < T;  // tokens past the prompt do not decay the state
      *reinterpret_cast<float4*>(&sh.cc[tok * CS + seg * 4]) =
          make_float4(ok ? chunk_log2_decay(nd[i].x) : 0.f, ok ? chunk_log2_decay(nd[i].y) : 0.f,
                      ok ? chunk_log2_decay(nd[i].z) : 0.f, ok ? chunk_log2_decay(nd[i].w) : 0.f);
    }
    if (t0 + C < T) fetch(t0 + C);
    __syncthreads();

    // ---- 2. prefix sums of the log2 decays over the chunk's tokens
    prefix_over_tokens<DK, CS>(sh.cc, sh.glast, tid);
    __syncthreads();

    // ---- 3. R o G_prev and K o G_C / G (token rows), split; the bonus diagonal;
    //         thread (token, 8-channel segment)
    for (int pc = tid; pc < C * KP; pc += kThreads) {
      const int tok = pc / KP, seg = pc % KP;
      float kf[8], rf[8], cf[8], cp[8], cl[8];
      unpack8(*reinterpret_cast<const uint4*>(&sh.k[tok * KS + seg * 8]), kf);
      unpack8(*reinterpret_cast<const uint4*>(&sh.q[tok * KS + seg * 8]), rf);
      load8(&sh.cc[tok * CS + seg * 8], cf);
      if (tok > 0) load8(&sh.cc[(tok - 1) * CS + seg * 8], cp);  // G_{tok-1}
      else
#pragma unroll
        for (int e = 0; e < 8; ++e) cp[e] = 0.f;
      load8(&sh.cc[(C - 1) * CS + seg * 8], cl);
      uint32_t rh[4], rl[4], kdh2[4], kdl2[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {  // channels e, e + 1 packed
        split2(rf[e] * fexp2(cp[e]), rf[e + 1] * fexp2(cp[e + 1]), rh[e / 2], rl[e / 2]);
        split2(kf[e] * fexp2(cl[e] - cf[e]), kf[e + 1] * fexp2(cl[e + 1] - cf[e + 1]), kdh2[e / 2], kdl2[e / 2]);
      }
      st_kperm8(&sh.rgh[tok * KS], seg * 8, make_uint4(rh[0], rh[1], rh[2], rh[3]));
      st_kperm8(&sh.rgl[tok * KS], seg * 8, make_uint4(rl[0], rl[1], rl[2], rl[3]));
      *reinterpret_cast<uint4*>(&sh.kdh[tok * RS + seg * 8]) = make_uint4(kdh2[0], kdh2[1], kdh2[2], kdh2[3]);
      *reinterpret_cast<uint4*>(&sh.kdl[tok * RS + seg * 8]) = make_uint4(kdl2[0], kdl2[1], kdl2[2], kdl2[3]);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(rf[e] * sh.bonus[seg * 8 + e], kf[e], d);
      d = group_sum<KP>(d);
      if (seg == 0) sh.pd[tok] = d;
    }

    // ---- 4. P (see the KDA kernel for the reference-token split; rows use G_{i-1})
    bool direct;
    {
      bool big = false;
      for (int ch = tid; ch < DK; ch += kThreads)
        big = big || -sh.cc[15 * CS + ch] > 60.f || sh.cc[15 * CS + ch] - sh.cc[(C - 1) * CS + ch] > 60.f;
      direct = __syncthreads_or(big);  // also orders step 3's stores before the reads below
    }
    if (!direct) {
      // wave w: channel steps kk = w % 2, w % 2 + 2, ...; waves 0, 1 the block (0,0), waves
      // 2, 3 the blocks (1,0) and (1,1), so each row and column operand is built once; the
      // two partial sums per entry are added in a fixed order through LDS
      constexpr int NKS = DK / 32, NKW = NKS < 2 ? NKS : 2;
      const int ks0 = wave & 1;
      const bool top = wave < 2;
      f32x4 acc[3];  // blocks (0,0), (1,0), (1,1)
#pragma unroll
      for (int m = 0; m < 3; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
      auto ops = [](const uint32_t (&w)[3][4], bf16x8 (&x)[3]) {
#pragma unroll
        for (int u = 0; u < 3; ++u) x[u] = pack8(w[u][0], w[u][1], w[u][2], w[u][3]);
      };
      for (int kk = ks0; kk < NKS; kk += 2) {
        const int ch0 = 32 * kk + 8 * lg;
        float k0[8], c0[8];
        unpack8(*reinterpret_cast<const uint4*>(&sh.k[ln * KS + ch0]), k0);
        load8(&sh.cc[ln * CS + ch0], c0);
        if (top) {  // rows: r of token ln with G_{ln-1} (R = start); columns: token ln (R = start)
          float cp[8], r0[8];
          if (ln > 0) load8(&sh.cc[(ln - 1) * CS + ch0], cp);
          else
#pragma unroll
            for (int e = 0; e < 8; ++e) cp[e] = 0.f;
          unpack8(*reinterpret_cast<const uint4*>(&sh.q[ln * KS + ch0]), r0);
          uint32_t ra[3][4], c00[3][4];
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            split3(r0[e] * fexp2(cp[e]), r0[e + 1] * fexp2(cp[e + 1]), ra[0][e / 2], ra[1][e / 2], ra[2][e / 2]);
            split3(k0[e] * fexp2(-c0[e]), k0[e + 1] * fexp2(-c0[e + 1]), c00[0][e / 2], c00[1][e / 2],
                   c00[2][e / 2]);
          }
          bf16x8 RA[3], C00[3];
          ops(ra, RA);
          ops(c00, C00);
          acc[0] = mma3(RA, C00, acc[0]);
        } else {  // rows: token 16 + ln with G_{15 + ln} (R = 15); columns: tokens ln, 16 + ln (R = 15)
          float ref[8], cp[8], c1[8], k1[8], r1[8];
          load8(&sh.cc[15 * CS + ch0], ref);
          load8(&sh.cc[(15 + ln) * CS + ch0], cp);
          load8(&sh.cc[(16 + ln) * CS + ch0], c1);
          unpack8(*reinterpret_cast<const uint4*>(&sh.k[(16 + ln) * KS + ch0]), k1);
          unpack8(*reinterpret_cast<const uint4*>(&sh.q[(16 + ln) * KS + ch0]), r1);
          uint32_t rb[3][4], c10[3][4], c11[3][4];
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            split3(r1[e] * fexp2(cp[e] - ref[e]), r1[e + 1] * fexp2(cp[e + 1] - ref[e + 1]), rb[0][e / 2],
                   rb[1][e / 2], rb[2][e / 2]);
            split3(k0[e] * fexp2(ref[e] - c0[e]), k0[e + 1] * fexp2(ref[e + 1] - c0[e + 1]), c10[0][e / 2],
                   c10[1][e / 2], c10[2][e / 2]);
            split3(k1[e] * fexp2(ref[e] - c1[e]), k1[e + 1] * fexp2(ref[e + 1] - c1[e + 1]), c11[0][e / 2],
                   c11[1][e / 2], c11[2][e / 2]);
          }
          bf16x8 RB[3], C10[3], C11[3];
          ops(rb, RB);
          ops(c10, C10);
          ops(c11, C11);
          acc[1] = mma3(RB, C10, acc[1]);
          acc[2] = mma3(RB, C11, acc[2]);
        }
      }
      __syncthreads();  // part overlays cc
      if (ks0 < NKW) {  // part[channel-step slot][block][r][lane]
#pragma unroll
        for (int m = 0; m < 3; ++m) {
          if (top != (m == 0)) continue;
#pragma unroll
          for (int r = 0; r < 4; ++r) sh.part[((ks0 * 3 + m) * 4 + r) * 64 + lane] = acc[m][r];
        }
      }
      __syncthreads();
      // thread (r = wave, lane): entry r of this lane in each block; the upper right block is zero
      const int r = wave;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int ib = m == 0 || m == 3 ? 0 : 1, jb = m >= 2 ? 1 : 0;  // (0,0), (1,0), (1,1), (0,1)
        const int i = 16 * ib + 4 * lg + r, j = 16 * jb + ln;
        float pm = 0.f;
        if (m < 3) {
          float sum = 0.f;
#pragma unroll
          for (int w = 0; w < NKW; ++w) sum += sh.part[((w * 3 + m) * 4 + r) * 64 + lane];
          pm = j < i ? sum : j == i ? sh.pd[i] : 0.f;
        }
        uint32_t hi, lo;
        split2(pm, 0.f, hi, lo);
        sh.pmh[i * TB + j] = static_cast<uint16_t>(hi);
        sh.pml[i * TB + j] = static_cast<uint16_t>(lo);
      }
    } else {
      // pairwise: thread (row pair ip, 31 - ip; channel slice sl); j < row, plus the diagonal
      constexpr int SL = DK / 16;
      const int ip = tid >> 4, sl = tid & 15;
      for (int e = tid; e < C * C; e += kThreads) {
        const int i = e / C, jj = e % C;
        if (jj >= i) {
          uint32_t hi, lo;
          split2(jj == i ? sh.pd[i] : 0.f, 0.f, hi, lo);
          sh.pmh[i * TB + jj] = static_cast<uint16_t>(hi);
          sh.pml[i * TB + jj] = static_cast<uint16_t>(lo);
        }
      }
      float rr[2][SL], cr[2][SL];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int r = w == 0 ? ip : C - 1 - ip;
#pragma unroll
        for (int e = 0; e < SL; ++e) {
          rr[w][e] = bf16_to_f32(sh.q[r * KS + sl * SL + e]);
          cr[w][e] = r > 0 ? sh.cc[(r - 1) * CS + sl * SL + e] : 0.f;
        }
      }
      for (int n = 0; n < C - 1; ++n) {  // row ip takes j = 0..ip-1, row 31 - ip takes j = 0..30 - ip
        const bool first = n < ip;
        const int r = first ? ip : C - 1 - ip, j = first ? n : n - ip;
        float pv = 0.f;
#pragma unroll
        for (int e = 0; e < SL; ++e) {
          const float u = bf16_to_f32(sh.k[j * KS + sl * SL + e]) *
                          fexp2((first ? cr[0][e] : cr[1][e]) - sh.cc[j * CS + sl * SL + e]);
          pv = fmaf(first ? rr[0][e] : rr[1][e], u, pv);
        }
        pv = group_sum<16>(pv);
        if (sl == 0) {
          uint32_t hi, lo;
          split2(pv, 0.f, hi, lo);
          sh.pmh[r * TB + j] = static_cast<uint16_t>(hi);
          sh.pml[r * TB + j] = static_cast<uint16_t>(lo);
        }
      }
    }
    __syncthreads();

    // ---- 5. O^T = S^T (R o G_prev)^T + V^T P^T (the operands swapped: each lane holds four
    //         adjacent columns of one token, token 16 ib + ln, columns 16 cb + 4 lg .. + 3)
    float O[2][NCB][4];
    {
      f32x4 qs[2][NCB];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) qs[ib][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kp = 0; kp < NKP; ++kp) {
        // S is replaced by diag(G_C) S (the first term of the update in step 6) as it is
        // split, so the split consumes the old S
        bf16x8 shi[NCB], slo[NCB];
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(&sh.glast[32 * kp + 4 * lg]);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(&sh.glast[32 * kp + 16 + 4 * lg]);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          float x0[4], x1[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x0[r] = S[2 * kp][cb][r];
            x1[r] = S[2 * kp + 1][cb][r];
            S[2 * kp][cb][r] = g0[r] * x0[r];
            S[2 * kp + 1][cb][r] = g1[r] * x1[r];
          }
          split_pair(x0, x1, shi[cb], slo[cb]);
        }
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
          const int rowk = (16 * ib + ln) * KS + 32 * kp + 8 * lg;  // channels 32 kp + 4 lg + {0..3, 16..19}
          const bf16x8 rah = ld_b128(&sh.rgh[rowk]), ral = ld_b128(&sh.rgl[rowk]);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            qs[ib][cb] = mma(shi[cb], rah, qs[ib][cb]);
            qs[ib][cb] = mma(slo[cb], rah, qs[ib][cb]);
            qs[ib][cb] = mma(shi[cb], ral, qs[ib][cb]);
          }
        }
      }
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) O[ib][cb][r] = qs[ib][cb][r];
    }
    const auto orows = out_rows(a.out, bseq, T, H, DV, t0, C);
    const uint32_t olane = static_cast<uint32_t>((ln * H + static_cast<int>(h)) * DV + col0 + 4 * lg) * 4;
    bf16x8 vb[NCB];  // V[token 8 lg + s][this lane's column]: the A operand of V^T P^T, the B operand of the update
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      vb[cb] = ld_tr8(sh.v, VS, 8 * lg, 8 * lg + 4, col0 + 16 * cb, ln);
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      const bf16x8 pah = ld_b128(&sh.pmh[(16 * ib + ln) * TB + 8 * lg]);
      const bf16x8 pal = ld_b128(&sh.pml[(16 * ib + ln) * TB + 8 * lg]);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        f32x4 acc = {O[ib][cb][0], O[ib][cb][1], O[ib][cb][2], O[ib][cb][3]};
        acc = mma(vb[cb], pah, acc);
        acc = mma(vb[cb], pal, acc);
        st_out4(orows, olane + static_cast<uint32_t>(16 * ib * H * DV + 16 * cb) * 4, acc);
      }
    }

    // ---- 6. S = diag(G_C) S + (K o G_C / G)^T V, diag(G_C) S formed in step 5
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const bf16x8 kah = ld_tr8(sh.kdh, RS, 8 * lg, 8 * lg + 4, 16 * kb, ln);  // tokens 8 lg .. 8 lg + 7
      const bf16x8 kal = ld_tr8(sh.kdl, RS, 8 * lg, 8 * lg + 4, 16 * kb, ln);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        f32x4 acc = {S[kb][cb][0], S[kb][cb][1], S[kb][cb][2], S[kb][cb][3]};
        acc = mma(kah, vb[cb], acc);
        acc = mma(kal, vb[cb], acc);
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
      for (int r = 0; r < 4; ++r) st_base<BF>(brsrc, bvoff, ((16 * kb + r) * DV + 16 * cb) * EB, S[kb][cb][r]);
}

}  // namespace

hipError_t launch_prefill(int variant, bool bf16_base, int dk, int dv, int tiles, const PoolArgs& p,
                          const PrefillArgs& a, hipStream_t stream) {
#define DL_PREFILL(BF_, DK_, DV_)                                                   \
  do {                                                                              \
    if (variant == DL_KDA) prefill_kda_kernel<DK_, DV_, BF_><<<tiles, kda_threads<DV_>(), 0, stream>>>(p, a); \
    else if (variant == DL_RWKV6) prefill_rwkv_kernel<DK_, DV_, BF_><<<tiles, kThreads, 0, stream>>>(p, a); \
    else prefill_kernel<DK_, DV_, BF_><<<tiles, gdn_threads<DV_>(), 0, stream>>>(p, a);        \
  } while (0)
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
