// Device helpers shared by the hybrid-block kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs2 {

constexpr int kHeads = 16;     // query heads sharing the one KV head (MQA)
constexpr int kDim = 128;      // head_dim
constexpr int kWindow = 128;   // recent positions always selected
constexpr int kTopK = 1024;    // positions selected before the window
constexpr int kBudget = kWindow + kTopK;
// One split-K partial: running max m[16] and sum z[16] (log2 domain), then the
// unnormalised output O[16][128].
constexpr int kPartialFloats = 2 * kHeads + kHeads * kDim;

// Rows [base, base + len) of sequence b, clamped so that any seq_offsets
// stays inside the N cache rows and within max_context.
__device__ __forceinline__ void seq_bounds(const int64_t* offs, int b, int64_t total, int64_t max_ctx,
                                           int64_t& base, int& len) {
  int64_t a = offs[b];
  int64_t e = offs[b + 1];
  a = a < 0 ? 0 : (a > total ? total : a);
  e = e < a ? a : (e > total ? total : e);
  if (e - a > max_ctx) e = a + max_ctx;
  base = a;
  len = static_cast<int>(e - a);
}

// Work item wg of a 1-D grid over the items of a ragged batch, numbered
// sequence by sequence, count(len) items for a sequence of len tokens: the
// sequence b of the item and its index j there.  A 2-D grid sized by the
// longest sequence would dispatch every hole as a workgroup that loads its
// bounds and exits.  Every lane of the wave computes the same answer (a wave
// prefix over 64 sequences at a time); false past the last item.
template <class CountFn>
__device__ bool find_item(const int64_t* offs, int batch, int64_t total, int64_t max_ctx, int wg, CountFn count,
                          int& b, int& j) {
  const int lane = threadIdx.x & 63;
  int carry = 0;  // items of the sequences before this pass
  for (int s0 = 0; s0 < batch; s0 += 64) {
    const int sb = s0 + lane;
    int64_t sbase = 0;
    int slen = 0;
    if (sb < batch) seq_bounds(offs, sb, total, max_ctx, sbase, slen);
    const int nb = sb < batch ? count(slen) : 0;
    int incl = nb;  // inclusive prefix sum over the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    const int tot = __shfl(incl, 63);
    if (wg < carry + tot) {
      const uint64_t hit = __ballot(carry + incl > wg);
      const int src = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      b = s0 + src;
      j = wg - carry - __shfl(incl - nb, src);
      return true;
    }
    carry += tot;
  }
  return false;
}

// Number of selected rows of a sequence, clamped to what the sequence can hold.
__device__ __forceinline__ int clamp_count(int count, int len, int budget) {
  const int cap = len < budget ? len : budget;
  return count < 0 ? 0 : (count > cap ? cap : count);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// D[16x16] += A[16x32] B[32x16], bf16 inputs, fp32 accumulate.  Lane l holds
// row (l % 16) of A and column (l % 16) of B, each with 8 values of the
// reduction index; D row 4*(l/16)+i, column l%16 is element i.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D[16x16] += A[16x4] B[4x16] in fp32.  Lane l holds A[l%16][l/16] and
// B[l/16][l%16]; D row 4*(l/16)+i, column l%16 is element i.
__device__ __forceinline__ f32x4 mfma_f32_16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// D[16x16] += A[16x16] B[16x16], bf16 inputs, fp32 accumulate.  Lane l holds
// row (l % 16) of A and column (l % 16) of B, each with the 4 values of the
// reduction index 4*(l/16) .. 4*(l/16)+3; D as above.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma_bf16_16x16x16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                  0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// fp32 -> OCP E4M3 code (1 sign, 4 exponent bits with bias 7, 3 mantissa
// bits; exponent field 0 holds the subnormals m * 2^-9; no infinities, and
// S.1111.111 is NaN, so the largest finite value is 448): round to nearest,
// ties to the even code, magnitudes above 448 (and NaN) saturate to +-448.
// Branch-free: from 2^-6 up, the fp32 bit pattern rounded at its 20th bit is
// the code with the exponent bias 127 in place of 7 (the carry of a mantissa
// that rounds up moves into the exponent); below 2^-6 the code is the
// magnitude in units of 2^-9, rounded (a code of 8 is the smallest normal).
__device__ __forceinline__ uint32_t f32_to_e4m3_rne_sat(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t mag = u & 0x7FFFFFFFu;
  const uint32_t normal = ((mag + 0x7FFFFu + ((mag >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
  const uint32_t sub = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(mag) * 512.f));
  const uint32_t code = mag < 0x3C800000u ? sub : min(normal, 0x7Eu);  // 0x3C800000 = 2^-6
  return ((u >> 24) & 0x80u) | code;
}

// 64-bit lane exchange: the value of lane (lane ^ m).
__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m);
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// Byte permute of the pair {hi_word, lo_word}: selector byte i picks byte
// sel_i of the 8-byte value lo_word | hi_word << 32.
__device__ __forceinline__ uint32_t perm(uint32_t hi_word, uint32_t lo_word, uint32_t sel) {
  return __builtin_amdgcn_perm(hi_word, lo_word, sel);
}
constexpr uint32_t kLoHalves = 0x05040100u;  // (lo_word.lo16, hi_word.lo16)
constexpr uint32_t kHiHalves = 0x07060302u;  // (lo_word.hi16, hi_word.hi16)

// Split an fp32 value into three bfloat16 parts whose exact sum is the value:
// each part keeps the top 8 significant bits of what the previous parts left,
// by truncation, so the subtractions are exact and 3 x 8 bits cover binary32's
// 24-bit significand.  Products of a part with a bf16 (or E4M3) key are exact
// in fp32, so three bf16 MFMAs give an fp32-accurate dot product.
__device__ __forceinline__ void split3(float x, uint32_t& h, uint32_t& m, uint32_t& l) {
  const uint32_t hu = __float_as_uint(x) & 0xFFFF0000u;
  const float r1 = x - __uint_as_float(hu);
  const uint32_t mu = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(mu);
  const uint32_t lu = __float_as_uint(r2) & 0xFFFF0000u;
  h = hu >> 16;
  m = mu >> 16;
  l = lu >> 16;
}

// Reduction-dim layout of S^T = K Q^T on the 16x16x32 MFMA.  Lane (n = l%16,
// g = l/16) holds, for k-step s = 0..3, eight consecutive dims starting at
// kdim0(s, g) of token n (K operand) and of head n (Q operand).  The layout is
// chosen so each 16-byte K load instruction of a wave reads 64 contiguous
// bytes of every row: bf16 step s, group g -> dims 32s + 8g; E4M3 (one 16-byte
// load per two steps) -> dims 64(s/2) + 16g + 8(s%2).
template <bool FP8>
__device__ __forceinline__ int kdim0(int s, int g) {
  return FP8 ? 64 * (s >> 1) + 16 * g + 8 * (s & 1) : 32 * s + 8 * g;
}

// Three bf16 parts of (q * qscale) for 8 query values (those of one k-step
// and lane group, see load_q8).
__device__ __forceinline__ void split_q8(const float4& a, const float4& c, float qscale, u32x4& ph, u32x4& pm,
                                         u32x4& pl) {
  const float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t h0, m0, l0, h1, m1, l1;
    split3(x[2 * i] * qscale, h0, m0, l0);
    split3(x[2 * i + 1] * qscale, h1, m1, l1);
    ph[i] = h0 | (h1 << 16);
    pm[i] = m0 | (m1 << 16);
    pl[i] = l0 | (l1 << 16);
  }
}

// The eight query values of k-step s for lane group g (raw fp32).  Loaded
// apart from their split so that callers can issue these loads ahead of the
// first tile's: a wait for data counts loads in issue order.
template <bool FP8>
__device__ __forceinline__ void load_q8(const float* __restrict__ q_head, int s, int g, float4& a, float4& c) {
  const float* src = q_head + kdim0<FP8>(s, g);
  a = *reinterpret_cast<const float4*>(src);
  c = *reinterpret_cast<const float4*>(src + 4);
}

// Query operand held in registers (one wave's own query).
struct QRegs {
  bf16x8 part[3][4];
  __device__ __forceinline__ bf16x8 get(int p, int s) const { return part[p][s]; }
};
struct QRaw {
  float4 a[4], c[4];
};
template <bool FP8>
__device__ __forceinline__ void load_qraw(const float* __restrict__ q_head, int g, QRaw& r) {
#pragma unroll
  for (int s = 0; s < 4; ++s) load_q8<FP8>(q_head, s, g, r.a[s], r.c[s]);
}
__device__ __forceinline__ void qregs_from(const QRaw& r, float qscale, QRegs& f) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u32x4 ph, pm, pl;
    split_q8(r.a[s], r.c[s], qscale, ph, pm, pl);
    f.part[0][s] = as_bf16x8(ph);
    f.part[1][s] = as_bf16x8(pm);
    f.part[2][s] = as_bf16x8(pl);
  }
}

// Query operand shared by a workgroup's waves through LDS: s_q[(p*4 + s)*64 + lane].
constexpr int kQLdsVecs = 3 * 4 * 64;
struct QShared {
  const u32x4* s_q;
  int lane;
  __device__ __forceinline__ bf16x8 get(int p, int s) const { return as_bf16x8(s_q[(p * 4 + s) * 64 + lane]); }
};

// Build the LDS query operand of heads [16][128] with 256 threads: the raw
// loads (thread t: k-step t / 64), then the split and the LDS stores.
template <bool FP8>
__device__ __forceinline__ void load_q_lds_raw(const float* __restrict__ q_heads, float4& a, float4& c) {
  const int lane = threadIdx.x & 63;
  load_q8<FP8>(q_heads + (lane & 15) * kDim, threadIdx.x >> 6, lane >> 4, a, c);
}
__device__ __forceinline__ void store_q_lds(const float4& a, const float4& c, float qscale, u32x4* s_q) {
  const int s = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  u32x4 ph, pm, pl;
  split_q8(a, c, qscale, ph, pm, pl);
  s_q[(0 * 4 + s) * 64 + lane] = ph;
  s_q[(1 * 4 + s) * 64 + lane] = pm;
  s_q[(2 * 4 + s) * 64 + lane] = pl;
}
template <bool FP8>
__device__ __forceinline__ void build_q_lds(const float* __restrict__ q_heads, float qscale, u32x4* s_q) {
  float4 a, c;
  load_q_lds_raw<FP8>(q_heads, a, c);
  store_q_lds(a, c, qscale, s_q);
}

// Row byte offset of the j-th 16-byte K load of lane group g (bf16: j = s,
// four loads; E4M3: j = s/2, two loads), matching kdim0.
__device__ __forceinline__ int kload_offset(int j, int g) { return 64 * j + 16 * g; }

// Two OCP E4M3 codes (bytes 0,1 or 2,3 of w) -> two bf16 packed in a word.
// The conversion to fp32 is exact and E4M3 has 4 significant bits, so taking
// the upper half of each fp32 word is exact too.
template <bool HIGH_PAIR>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  const f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8(w, HIGH_PAIR);
  return perm(__float_as_uint(f[1]), __float_as_uint(f[0]), kHiHalves);
}

// 16 E4M3 codes -> 16 bf16 (two bf16x8 operands).
__device__ __forceinline__ void e4m3x16_to_bf16(u32x4 w, bf16x8& lo, bf16x8& hi) {
  u32x4 a, b;
  a[0] = e4m3x2_to_bf16x2<false>(w[0]);
  a[1] = e4m3x2_to_bf16x2<true>(w[0]);
  a[2] = e4m3x2_to_bf16x2<false>(w[1]);
  a[3] = e4m3x2_to_bf16x2<true>(w[1]);
  b[0] = e4m3x2_to_bf16x2<false>(w[2]);
  b[1] = e4m3x2_to_bf16x2<true>(w[2]);
  b[2] = e4m3x2_to_bf16x2<false>(w[3]);
  b[3] = e4m3x2_to_bf16x2<true>(w[3]);
  lo = as_bf16x8(a);
  hi = as_bf16x8(b);
}

// Online-softmax state of one wave for 16 heads: lane (n, g) keeps head n's
// reference max m (log2 domain; at most kRescaleSlack below the running max),
// its lane-group share of the sum z of exp2(l - m), and the unnormalised
// output O^T tile: o[t][i] = O[head n][dim 32g + 8i + t], all relative to m.
struct SoftmaxState {
  float m;
  float z;
  f32x4 o[8];
};

__device__ __forceinline__ void softmax_init(SoftmaxState& st) {
  st.m = -INFINITY;
  st.z = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) st.o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// O^T += V^T P^T for one tile of 16 tokens on bf16 MFMA (16x16x16).
// Reduction index = the tile's tokens.  MFMA j serves dims 8m + j (A row m),
// so lane (m, g) needs V[4g + r][8m + j] for r = 0..3: its own four V loads,
// regrouped by byte permutes (no data crosses lanes).  The B operand is the
// lane's own four probabilities.  P (times the per-token V scale) is split
// into a bf16 head and a bf16 tail, so the product keeps 16 significant bits
// of each weight (V itself is exact in bf16); MFMA j leaves
// O[head n][dim 32g + 8i + j] in element i of st.o[j] on lane (n, g).
// Operands of O^T += V^T P^T for one tile: ph / pl the bf16 head and tail
// of the lane's four weights (tokens 4g .. 4g + 3), a[j] the lane's V values
// of dim 8n + j for those tokens (MFMA j's A operand, row n).
// The P operand of a tile's P.V (p[r]: weight of token 4g + r, times its V
// scale for E4M3): bf16 head ph and exact bf16 tail pl.
template <bool FP8>
__device__ __forceinline__ void pv_p_operand(const float (&p)[4], const float (&vscale)[4], u32x2& ph, u32x2& pl) {
  float w[4], tail[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    w[r] = FP8 ? p[r] * vscale[r] : p[r];
    tail[r] = w[r] - __uint_as_float(__float_as_uint(w[r]) & 0xFFFF0000u);  // exact
  }
  ph = u32x2{perm(__float_as_uint(w[1]), __float_as_uint(w[0]), kHiHalves),
             perm(__float_as_uint(w[3]), __float_as_uint(w[2]), kHiHalves)};
  pl = u32x2{perm(__float_as_uint(tail[1]), __float_as_uint(tail[0]), kHiHalves),
             perm(__float_as_uint(tail[3]), __float_as_uint(tail[2]), kHiHalves)};
}

// The V operand of a tile's P.V: a[j] holds dims 16 j' .. of the tile's V^T
// in the 16x16x16 A layout (one query's weights or several queries' share it).
template <bool FP8>
__device__ __forceinline__ void pv_v_operand(const u32x4 (&vraw)[4], u32x2 (&a)[8]) {
  if constexpr (FP8) {
    // codes of dims 4h .. 4h + 3 sit in word h of each token's load
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const uint32_t t0 = vraw[2 * pr][h], t1 = vraw[2 * pr + 1][h];
        // interleave the two tokens' codes: (t0.d, t1.d, t0.d+1, t1.d+1)
        const uint32_t x01 = perm(t1, t0, 0x05010400u);
        const uint32_t x23 = perm(t1, t0, 0x07030602u);
        a[4 * h + 0][pr] = e4m3x2_to_bf16x2<false>(x01);
        a[4 * h + 1][pr] = e4m3x2_to_bf16x2<true>(x01);
        a[4 * h + 2][pr] = e4m3x2_to_bf16x2<false>(x23);
        a[4 * h + 3][pr] = e4m3x2_to_bf16x2<true>(x23);
      }
    }
  } else {
    // word i of a token's load holds dims 2i (low half) and 2i + 1 (high half)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const uint32_t t0 = vraw[2 * pr][i], t1 = vraw[2 * pr + 1][i];
        a[2 * i][pr] = perm(t1, t0, kLoHalves);
        a[2 * i + 1][pr] = perm(t1, t0, kHiHalves);
      }
    }
  }
}

template <bool FP8>
__device__ __forceinline__ void pv_operands(const u32x4 (&vraw)[4], const float (&p)[4], const float (&vscale)[4],
                                            u32x2 (&a)[8], u32x2& ph, u32x2& pl) {
  pv_p_operand<FP8>(p, vscale, ph, pl);
  pv_v_operand<FP8>(vraw, a);
}

template <bool FP8>
__device__ __forceinline__ void pv_tile(const u32x4 (&vraw)[4], const float (&p)[4], const float (&vscale)[4],
                                        SoftmaxState& st) {
  u32x2 a[8], ph, pl;
  pv_operands<FP8>(vraw, p, vscale, a, ph, pl);
#pragma unroll
  for (int j = 0; j < 8; ++j) st.o[j] = mfma_bf16_16x16x16(a[j], ph, st.o[j]);
#pragma unroll
  for (int j = 0; j < 8; ++j) st.o[j] = mfma_bf16_16x16x16(a[j], pl, st.o[j]);
}

// Two tiles' O^T += V^T P^T on the 16x16x32 MFMA, which reduces over 32
// tokens at the cost of one 16x16x16: reduction index 8g + r is token
// 4g + r of the first tile for r < 4 and of the second for r >= 4, so each
// lane's operands are its own two tiles' values, concatenated.
template <bool FP8>
__device__ __forceinline__ void pv_tiles2(const u32x4 (&v0)[4], const float (&p0)[4], const float (&s0)[4],
                                          const u32x4 (&v1)[4], const float (&p1)[4], const float (&s1)[4],
                                          SoftmaxState& st) {
  u32x2 a0[8], a1[8], ph0, pl0, ph1, pl1;
  pv_operands<FP8>(v0, p0, s0, a0, ph0, pl0);
  pv_operands<FP8>(v1, p1, s1, a1, ph1, pl1);
  const bf16x8 ph = as_bf16x8(u32x4{ph0[0], ph0[1], ph1[0], ph1[1]});
  const bf16x8 pl = as_bf16x8(u32x4{pl0[0], pl0[1], pl1[0], pl1[1]});
  bf16x8 a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = as_bf16x8(u32x4{a0[j][0], a0[j][1], a1[j][0], a1[j][1]});
#pragma unroll
  for (int j = 0; j < 8; ++j) st.o[j] = mfma_bf16_16x16x32(a[j], ph, st.o[j]);
#pragma unroll
  for (int j = 0; j < 8; ++j) st.o[j] = mfma_bf16_16x16x32(a[j], pl, st.o[j]);
}

// The second half of attend_tile (below): the online-softmax update and P.V
// from the tile's S^T = K Q^T in s (lane (n, g): head n, tokens 4g + r).  A
// caller with several queries per tile forms their products as interleaved
// MFMA chains and then calls this once per query.
template <bool FP8>
__device__ __forceinline__ void tile_update(const f32x4& s, const u32x4 (&vraw)[4], const float (&kscale)[4],
                                            const float (&vscale)[4], int nvalid, int g, SoftmaxState& st,
                                            float (&lg)[4], float (&p)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) lg[r] = (4 * g + r < nvalid) ? s[r] * kscale[r] : -INFINITY;
  float mx = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  // Lazy rescaling: a head keeps its reference max until a tile exceeds it by
  // more than kRescaleSlack (log2 units), so weights stay <= 2^kRescaleSlack and
  // the accumulators are rescaled only a few times per wave instead of at
  // nearly every tile.  Every partial carries its reference, so the math is
  // unchanged.
  constexpr float kRescaleSlack = 8.f;
  const bool raise = mx > st.m + kRescaleSlack;  // true on a head's first tile (m = -inf)
  if (__any(raise)) {
    const float mn = raise ? mx : st.m;
    const float alpha = __builtin_amdgcn_exp2f(st.m - mn);  // 0 on the first tile, 1 if unchanged
    st.z *= alpha;
#pragma unroll
    for (int t = 0; t < 8; ++t) st.o[t] *= alpha;
    st.m = mn;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(lg[r] - st.m);
  st.z += (p[0] + p[1]) + (p[2] + p[3]);
  pv_tile<FP8>(vraw, p, vscale, st);
}

// One tile of 16 context tokens for 16 heads.
//  kf[s]: K operand, lane (n, g): token n, dims kdim0(s, g) + i (bf16)
//  vraw[r]: V values of token 4g + r, dims 8n .. 8n + 7, lane (n, g): eight
//           bf16 (16 bytes) or eight E4M3 codes (first 8 bytes)
//  kscale[r], vscale[r]: per-token scales of token 4g + r (1 for bf16)
//  nvalid: tokens of the tile that exist (1..16); others are masked out
// Returns the log2-domain logits of tokens 4g + r for head n in lg[r]
// (-inf where masked) and p[r] = exp2(lg[r] - st.m), st.m being the head's
// reference max after this tile (within kRescaleSlack of the true running max).
template <bool FP8, class QSrc>
__device__ __forceinline__ void attend_tile(const QSrc& q, const bf16x8 (&kf)[4], const u32x4 (&vraw)[4],
                                            const float (&kscale)[4], const float (&vscale)[4], int nvalid,
                                            int g, SoftmaxState& st, float (&lg)[4], float (&p)[4]) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int part = 0; part < 3; ++part) {
#pragma unroll
    for (int k = 0; k < 4; ++k) s = mfma_bf16_16x16x32(kf[k], q.get(part, k), s);
  }
  tile_update<FP8>(s, vraw, kscale, vscale, nvalid, g, st, lg, p);
}

// NT tiles of 16 context tokens at once for 16 heads: attend_tile's
// arithmetic with the tiles' S^T = K Q^T products computed as NT independent
// MFMA chains (interleaved, so the matrix core is not left waiting on one
// chain's latency) and one online-softmax update over the NT * 16 tokens.
// PARTS of the query's three exact bf16 parts enter the products: 3 gives
// fp32-accurate logits; 2 keeps 16 significant bits of the query (logits
// within ~2^-16 relative), enough where no selection depends on them.
// Operands per tile as attend_tile; vload(t, vraw, vscale) supplies tile t's
// V rows and scales after the products are formed (their registers then
// reuse the K operand's).  nvalid[t] <= 0 masks tile t entirely; at least one
// token of the NT tiles must exist.
template <bool FP8, int NT, int PARTS, class QSrc, class VLoad>
__device__ __forceinline__ void attend_tiles(const QSrc& q, const bf16x8 (&kf)[NT][4],
                                             const float (&kscale)[NT][4], const int (&nvalid)[NT], int g,
                                             SoftmaxState& st, VLoad vload) {
  f32x4 s[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int part = 0; part < PARTS; ++part) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int t = 0; t < NT; ++t) s[t] = mfma_bf16_16x16x32(kf[t][k], q.get(part, k), s[t]);
    }
  }
  float lg[NT][4];
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      lg[t][r] = (4 * g + r < nvalid[t]) ? s[t][r] * kscale[t][r] : -INFINITY;
      mx = fmaxf(mx, lg[t][r]);
    }
  }
  // As attend_tile, but the head's maximum over the four lane groups is
  // formed only when some lane's own maximum calls for a rescale: a head's
  // maximum exceeds the reference by the slack exactly when one of its lanes'
  // does, so the outcome is the same and the lane exchanges (LDS round trips)
  // are skipped on the tiles that do not raise the reference.
  constexpr float kRescaleSlack = 8.f;  // as in attend_tile
  if (__any(mx > st.m + kRescaleSlack)) {
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool raise = mx > st.m + kRescaleSlack;
    const float mn = raise ? mx : st.m;
    const float alpha = __builtin_amdgcn_exp2f(st.m - mn);
    st.z *= alpha;
#pragma unroll
    for (int t = 0; t < 8; ++t) st.o[t] *= alpha;
    st.m = mn;
  }
  float p[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) p[t][r] = __builtin_amdgcn_exp2f(lg[t][r] - st.m);
    st.z += (p[t][0] + p[t][1]) + (p[t][2] + p[t][3]);
  }
  // P V over pairs of tiles on the 16x16x32 MFMA; an odd last tile alone
#pragma unroll
  for (int t = 0; t + 1 < NT; t += 2) {
    u32x4 v0[4], v1[4];
    float s0[4], s1[4];
    vload(t, v0, s0);
    vload(t + 1, v1, s1);
    pv_tiles2<FP8>(v0, p[t], s0, v1, p[t + 1], s1, st);
  }
  if constexpr (NT % 2) {
    u32x4 v[4];
    float sc[4];
    vload(NT - 1, v, sc);
    pv_tile<FP8>(v, p[NT - 1], sc, st);
  }
}

// DPP lane moves within a row of 16 lanes (plain VALU, no LDS crossbar).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Four sums over the 16 lanes of a row at once (reduce-scatter): lane n ends
// with the row's total of x[n >> 2].  Mirroring the row pairs lane n with a
// lane of the other half: each keeps two of the four values and sends the
// other two.  Mirroring the half-row pairs the two quads of a half: each keeps
// one.  Two swaps inside the quad finish the sum.
__device__ __forceinline__ float row_sums4(const float (&x)[4], int n) {
  const bool hi8 = (n & 8) != 0;
  float k0 = hi8 ? x[2] : x[0], k1 = hi8 ? x[3] : x[1];
  k0 += dpp_move<0x140>(hi8 ? x[0] : x[2]);  // row_mirror
  k1 += dpp_move<0x140>(hi8 ? x[1] : x[3]);
  const bool hi4 = (n & 4) != 0;
  float v = hi4 ? k1 : k0;
  v += dpp_move<0x141>(hi4 ? k0 : k1);  // row_half_mirror
  v += dpp_move<0x4E>(v);               // quad_perm [2, 3, 0, 1]
  v += dpp_move<0xB1>(v);               // quad_perm [1, 0, 3, 2]
  return v;
}

// Reduce z over the four lane groups (every lane of head n gets the total).
__device__ __forceinline__ float reduce_z(float z) {
  z += __shfl_xor(z, 16);
  z += __shfl_xor(z, 32);
  return z;
}

}  // namespace hs2
