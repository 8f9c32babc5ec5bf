// Stage 1: LSH bucket ids, h(x) = argmax([xR; -xR]).
//
// "Reformer: The Efficient Transformer" (research summary), Key points, LSH
// attention bullet: each vector is hashed as the argmax of the concatenation
// of its rotation xR and the negation -xR.  Bucket k < b/2 is +(xR)_k and
// bucket b/2 + k is -(xR)_k; ties go to the lowest bucket index.
//
// Design for gfx950
//   * The projection x.R is a dense contraction (tokens x d) . (d x b/2), so
//     bf16 inputs run on MFMA.  R = R_hi + R_lo with R_hi = bf16(R): the main
//     term x.R_hi runs on v_mfma_f32_32x32x16_bf16 (bf16 x bf16 products are
//     exact in float32).  The correction x.R_lo, about 2^-9 of the result, runs
//     on v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in fp6 e2m3 and
//     an E8M0 scale per block of 32 features (of one rotation column, and of
//     one token), at a quarter of the cost of a bf16 pass.  Its error is
//     bounded per token (below), so decisions stay exact.  Float32 inputs use
//     a plain FMA kernel.
//   * The matrix product is computed transposed, D = R^T X^T, so that each lane
//     receives 16 projections of ONE token per 32x32 tile.  Every projection is
//     turned into an ordered 32-bit key with one and-or: the float's bits with
//     the sign cleared and a candidate code in the low mantissa bits.  A
//     running top-two of keys per lane takes a med3, a max and a max3 per two
//     values.  The sign is left out of the keys: a running maximum of the raw
//     float bits as signed integers (a max3 per two values) tells at the end
//     of the round whether the winner is positive -- it is exactly when that
//     maximum reaches the winner's magnitude.  The two lanes sharing a token
//     merge once per round.
//   * The top-two keys give the two leading candidates and their gap.  When the
//     gap is below twice a bound on the error of one projection, the
//     (position, round) is queued and a fix-up kernel re-decides it in float64
//     between those two candidates (or over all columns when even the leading
//     magnitude is within the bound, e.g. x = 0).  By Cauchy-Schwarz, with x6
//     and R_lo6 the fp6 operands, one projection is off by at most
//       |x| max_j |R_j - R_hi,j - R_lo6,j| + |x - x6| max_j |R_lo6,j|
//     plus float32 accumulation (below 2^-15 (|x| max_j |R_j| + |x6| max_j
//     |R_lo6,j|) for up to 256 products), plus the key truncation.  The column
//     maxima come from the set-up kernel, |x| and |x - x6| from the lanes that
//     convert x.
//   * Rotation fragments are pre-arranged in global memory in the exact order
//     the MFMA A operands want them, so the copy into LDS is a straight
//     coalesced memcpy and every wave reads 1 KB contiguous per fragment (no
//     bank conflicts).  Tiles are double-buffered through LDS.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>

namespace rlsh {

namespace {

constexpr float kTauRel = 1.0f / 4096.0f;   // FMA path: 2^-12 of |x|_2 * max_j |R_j|_2
constexpr float kAccRel = 1.0f / 32768.0f;  // MFMA path: float32 accumulation, 2^-15
constexpr int kHashThreads = 256;           // 4 wavefronts
constexpr int kStrips = 2;                  // 32-token strips per wavefront

// --------------------------------------------------------------- keys ----
// key = the float's bits with the sign cleared and bits 0..code_bits-1
// replaced by a candidate code.  Unsigned order of keys is the order of |p|
// truncated to (23 - code_bits) mantissa bits; codes make keys distinct.
__device__ __forceinline__ uint32_t make_key(float p, uint32_t keep_mask, uint32_t code) {
  return (__float_as_uint(p) & keep_mask) | code;
}

// v_med3_u32 written out, so that the compiler does not share its max(a, b)
// with the max3 of the same values and then lose the max3.
__device__ __forceinline__ uint32_t med3_u32(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Top-two of {k1 >= k2, a, b}: the largest is max3(k1, a, b), the second
// max(k2, med3(k1, a, b)).
__device__ __forceinline__ void top2_push2(uint32_t& k1, uint32_t& k2, uint32_t a, uint32_t b) {
  k2 = max(k2, med3_u32(k1, a, b));
  k1 = max(max(k1, a), b);
}

__device__ __forceinline__ uint32_t umed3(uint32_t a, uint32_t b, uint32_t c) {
  return max(min(a, b), min(max(a, b), c));
}

__device__ __forceinline__ void top2_push(uint32_t& k1, uint32_t& k2, uint32_t key) {
  k2 = umed3(k1, k2, key);
  k1 = max(k1, key);
}

__device__ __forceinline__ void top2_merge(uint32_t& k1, uint32_t& k2, uint32_t o1, uint32_t o2) {
  uint32_t n2 = max(min(k1, o1), max(k2, o2));
  k1 = max(k1, o1);
  k2 = n2;
}

__device__ __forceinline__ float key_magnitude(uint32_t key, uint32_t code_mask) {
  return __uint_as_float(key & ~code_mask);
}

// Queued (token, round) pairs live in one region per hash workgroup (capacity
// = its tokens x rounds), counted in LDS, so no global atomic is contended.
constexpr int kTokensPerBlock = 256;

struct NearTieList {
  int32_t* counts;    // per workgroup: number of queued entries
  int32_t* entries;   // 3 per entry: token, round | full<<31, c1 | c2<<16
  int cap;            // entries per workgroup region
  int* lds_count;     // the workgroup's counter in LDS (set inside the kernel)
};

__device__ __forceinline__ void push_near_tie(NearTieList lst, int tok, int round, bool full, int c1, int c2) {
  int idx = atomicAdd(lst.lds_count, 1);
  int32_t* e = lst.entries + 3 * (static_cast<size_t>(blockIdx.x) * lst.cap + idx);
  e[0] = tok;
  e[1] = round | (full ? static_cast<int>(0x80000000u) : 0);
  e[2] = (c1 & 0xffff) | (c2 << 16);
}

// Shared decision once a token's top-two keys and |x|_2 are known.
// tau_x bounds the error of the gap between two projections before key
// truncation, which is added here.  smax is the largest raw projection bit
// pattern as a signed integer (the largest positive projection, if any): the
// winner is positive exactly when smax reaches its truncated magnitude.  Were
// the winner negative while a positive projection reached that magnitude, the
// two would share a truncated magnitude, so the gap would be zero and the
// fix-up would decide.
__device__ __forceinline__ void decide_and_store(uint32_t k1, uint32_t k2, int32_t smax, int col1, int col2,
                                                 float tau_x, int code_bits, int half, int tok, int seq_len,
                                                 int n_rounds, int round, int32_t* buckets, NearTieList lst) {
  const uint32_t code_mask = (1u << code_bits) - 1u;
  float m1 = key_magnitude(k1, code_mask);
  float m2 = key_magnitude(k2, code_mask);
  float tau = tau_x + m1 * __uint_as_float((127u + code_bits - 22u) << 23);
  const bool positive = smax >= static_cast<int32_t>(k1 & ~code_mask);
  int bucket = col1 + (positive ? 0 : half);
  int bh = tok / seq_len, pos = tok - bh * seq_len;
  buckets[(static_cast<size_t>(bh) * n_rounds + round) * seq_len + pos] = bucket;
  bool full = !(m1 > tau);
  if (full || (m1 - m2) <= tau) push_near_tie(lst, tok, round, full, col1, col2);
}

// The float32 bounds assume that the products and partial sums that matter
// stay far above the float32 subnormal range (and that the sums of squares
// behind |x| do not underflow).  Below |x| = 2^-56 or max_j |R_j| = 2^-56
// that is not assured, so such a (position, round) is re-decided in float64
// over all columns (an infinite bound makes it a full re-decision).
__device__ __forceinline__ float guard_tiny(float tau, float xnorm, float cmax) {
  return (xnorm >= 0x1p-56f && cmax >= 0x1p-56f) ? tau : INFINITY;
}

// MFMA path: twice the per-projection bound (see the top of this file), with
// a 2^-10 margin for the float32 evaluation of the bound itself.
__device__ __forceinline__ float split_gap_bound(float xnorm, float xerr, float cmax, float rho1, float rho2) {
  const float acc = kAccRel * (xnorm * cmax + (xnorm + xerr) * rho2);
  return guard_tiny(2.0f * (xnorm * rho1 + xerr * rho2 + acc) * (1.0f + 1.0f / 1024.0f), xnorm, cmax);
}

// Column-norm maxima, per rotation tile, as float bits in
// [3][n_rounds][n_ctiles]: max_j |R_j|, max_j |R_j - R_hi,j - R_lo6,j|,
// max_j |R_lo6,j| over the tile's columns j.  The set-up kernel writes one
// entry per workgroup (no atomics, so no clearing pass); readers take the
// maximum over a round's tiles.
enum { kBoundCmax = 0, kBoundRes = 1, kBoundLo = 2, kBoundTerms = 3 };

// A round's maximum of one term; every lane of the wavefront must call it.
__device__ __forceinline__ float round_bound(const uint32_t* __restrict__ bound_bits, int term, int n_rounds,
                                             int n_ctiles, int round) {
  const uint32_t* p = bound_bits + (static_cast<size_t>(term) * n_rounds + round) * n_ctiles;
  uint32_t m = 0u;
  for (int t = lane_id(); t < n_ctiles; t += 64) m = max(m, p[t]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, shfl_xor_u(m, off));
  return __uint_as_float(m);
}

// ------------------------------------------------------ preparation ----

// sqrt of a float64 sum of squares as float, rounded up (one float rounding,
// at most 2^-24 relative, covered by the factor).
__device__ __forceinline__ uint32_t norm_bits_up(double sum) {
  return __float_as_uint(static_cast<float>(sqrt(sum)) * 1.0000005f);
}

// Largest value of each lane's group of 32 lanes into *dst (non-negative
// float bits).
__device__ __forceinline__ void max32_to(uint32_t bits, uint32_t* dst) {
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) bits = max(bits, static_cast<uint32_t>(__shfl_xor(static_cast<int>(bits), off, 32)));
  if ((threadIdx.x & 31) == 0) *dst = bits;
}

// fp6 e2m3 (1 sign, 2 exponent bits with bias 1, 3 mantissa bits): the
// magnitude codes 0..31 stand for c/8 below 2, 2 + (c-16)/4 below 4 and
// 4 + (c-24)/2 up to 7.5; bit 5 is the sign.  Round to nearest, ties to the
// even code, for |q| <= 7.5.
__device__ __forceinline__ uint32_t e2m3_code(float q) {
  const float m = fabsf(q);
  float c;
  if (m < 2.0f) c = rintf(m * 8.0f);
  else if (m < 4.0f) c = 16.0f + rintf((m - 2.0f) * 4.0f);
  else c = 24.0f + rintf((m - 4.0f) * 2.0f);
  return static_cast<uint32_t>(c) | (q < 0.0f ? 32u : 0u);
}

__device__ __forceinline__ float e2m3_value(uint32_t code) {
  const float c = static_cast<float>(code & 31u);
  const float m = c < 16.0f ? c * 0.125f : (c < 24.0f ? 2.0f + (c - 16.0f) * 0.25f : 4.0f + (c - 24.0f) * 0.5f);
  return (code & 32u) ? -m : m;
}

// Exponent E of the power of two that maps a block whose largest magnitude
// is m into the e2m3 range (m * 2^-E in (3.75, 7.5]), kept inside E8M0's.
__device__ __forceinline__ int e2m3_block_exp(float m) {
  if (!(m > 0.0f)) return 0;
  const int k = ilogbf(m);
  const int e = m <= ldexpf(1.875f, k) ? k - 2 : k - 1;
  return max(-127, min(e, 127));
}

// 32 codes packed as 6-bit fields, field e at bits 6e..6e+5 of six dwords.
__device__ __forceinline__ void put_e2m3(uint32_t (&w)[6], int e, uint32_t code) {
  const int bit = 6 * e;
  w[bit / 32] |= code << (bit % 32);
  if (bit % 32 > 26) w[bit / 32 + 1] |= code >> (32 - bit % 32);
}

// Fragment tile layout (16-byte units) for one (round, tile of 32 columns):
//   [ks * 64 + l], ks < D/16: bf16 R_hi[k][c], c = 32t + l%32,
//       k = 16ks + 8(l/32) + 0..7 (A operand of v_mfma_f32_32x32x16_bf16);
//   [D * 4 + (2kb + j) * 64 + l], kb < D/64, j = 0, 1: dwords 4j..4j+3 of the
//       lane's 8-dword A operand of fp6 MFMA step kb: dwords 0..5 hold
//       R_lo[k][c] * 2^-E, k = 64kb + 32(l/32) + e in 6-bit field e, dword 6
//       the block's E8M0 scale byte 127 + E, dword 7 zero.
// With fp6 operands the scaled MFMA pairs field e of lane l with field e of
// the B operand's lane of the same l/32, and each lane's 32 fields form one
// scale block whose scale that lane supplies.
template <int D>
struct FragTile {
  static constexpr int kHiSteps = D / 16;              // bf16 MFMA k-steps
  static constexpr int kLoSteps = D / 64;              // fp6 MFMA k-steps
  static constexpr int kHiVec = kHiSteps * 64;
  static constexpr int kVec = kHiVec + kLoSteps * 2 * 64;
};

// Per-call set-up, one workgroup per (tile of 32 rotation columns, round):
//  - (FRAG) the fragment tile above, with R_hi = bf16(R) (round to nearest
//    even), R_lo = R - R_hi (exact in float32) and a power of two 2^E per
//    block of 32 features of a column that puts its largest |R_lo| into
//    (3.75, 7.5];
//  - R transposed to float32 [round][column][k], so that the fix-up reads a
//    column as one contiguous row;
//  - per-round maxima over columns of |R_j|, and (FRAG) of
//    |R_j - R_hi,j - R_lo6,j| and |R_lo6,j| (float64 sums, rounded up).
template <int D, bool FRAG>
__global__ __launch_bounds__(256) void hash_prepare_kernel(const float* __restrict__ rot, int half, int n_rounds,
                                                           int n_ctiles, u32x4* __restrict__ frag,
                                                           float* __restrict__ rt, uint32_t* __restrict__ bound_bits,
                                                           int32_t* n_near_ties) {
  using FT = FragTile<D>;
  constexpr int kGroups = 8;               // k-ranges per column
  constexpr int kPerG = D / kGroups;       // 8 or 16 values
  constexpr int kLoUnits = D / 32;         // fp6 scale blocks per column
  __shared__ double part[kGroups][32];
  __shared__ double part_res[kLoUnits][32];
  __shared__ double part_lo[kLoUnits][32];
  __shared__ float tile_r[D][33];          // the tile's 32 columns (zero past half), one coalesced read
  const int t = blockIdx.x, r = blockIdx.y;
  const float* R = rot + static_cast<size_t>(r) * D * half;
  {
    // all loads in flight before the first LDS store (launched with 256 threads)
    constexpr int kPer = D * 32 / 256;
    const int cl = threadIdx.x % 32, c = 32 * t + cl;
    float v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = c < half ? R[static_cast<size_t>(threadIdx.x / 32 + 8 * i) * half + c] : 0.0f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) tile_r[threadIdx.x / 32 + 8 * i][cl] = v[i];
  }
  __syncthreads();
  auto rval = [&](int k, int cl) -> float { return tile_r[k][cl]; };
  auto lo_of = [](float v) -> float { return v - bf16_to_f32(f32_to_bf16_rne(v)); };
  if (FRAG) {
    u32x4* tile = frag + (static_cast<size_t>(r) * n_ctiles + t) * FT::kVec;
    for (int u = threadIdx.x; u < FT::kHiVec; u += blockDim.x) {
      const int ks = u / 64, l = u % 64;
      const int c = l & 31;
      const int k0 = 16 * ks + 8 * (l >> 5);
      u32x4 hi;
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        hi[e / 2] = static_cast<uint32_t>(f32_to_bf16_rne(rval(k0 + e, c))) |
                    (static_cast<uint32_t>(f32_to_bf16_rne(rval(k0 + e + 1, c))) << 16);
      tile[u] = hi;
    }
    // Two threads per scale block (kb, lane l): thread p takes fields
    // 16p..16p+15, which are exactly dwords 3p..3p+2 of the packed codes.
    for (int u = threadIdx.x; u < FT::kLoSteps * 128; u += blockDim.x) {
      const int blk = u >> 1, p = u & 1;
      const int kb = blk / 64, l = blk % 64;
      const int c = l & 31;
      const int k0 = 64 * kb + 32 * (l >> 5) + 16 * p;
      float lo[16];
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        lo[e] = lo_of(rval(k0 + e, c));
        m = fmaxf(m, fabsf(lo[e]));
      }
      m = fmaxf(m, __shfl_xor(m, 1, 64));   // partner thread: u ^ 1, same wavefront
      const int E = e2m3_block_exp(m);
      uint32_t w[6] = {0u, 0u, 0u, 0u, 0u, 0u};
      double s_res = 0.0, s_lo = 0.0;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t code = e2m3_code(ldexpf(lo[e], -E));
        put_e2m3(w, e, code);
        const double lo6 = ldexp(static_cast<double>(e2m3_value(code)), E);
        const double res = static_cast<double>(lo[e]) - lo6;
        s_res += res * res;
        s_lo += lo6 * lo6;
      }
      // w[0..2] hold this thread's 16 fields (dwords 3p..3p+2 of the block)
      const uint32_t first_of_partner = static_cast<uint32_t>(__shfl_xor(static_cast<int>(w[0]), 1, 64));
      s_res += __shfl_xor(s_res, 1, 64);
      s_lo += __shfl_xor(s_lo, 1, 64);
      if (p == 0)
        tile[FT::kHiVec + (2 * kb) * 64 + l] = u32x4{w[0], w[1], w[2], first_of_partner};
      else
        tile[FT::kHiVec + (2 * kb + 1) * 64 + l] = u32x4{w[1], w[2], static_cast<uint32_t>(127 + E), 0u};
      if (p == 0) {
        part_res[2 * kb + (l >> 5)][c] = s_res;
        part_lo[2 * kb + (l >> 5)][c] = s_lo;
      }
    }
  }
  const int cl = threadIdx.x & 31, g = threadIdx.x >> 5;
  const int c = 32 * t + cl;
  double acc = 0.0;
  if (c < half) {
    float v[kPerG];
#pragma unroll
    for (int i = 0; i < kPerG; ++i) {
      v[i] = rval(g * kPerG + i, cl);
      acc += static_cast<double>(v[i]) * static_cast<double>(v[i]);
    }
    f32x4* dst = reinterpret_cast<f32x4*>(rt + (static_cast<size_t>(r) * half + c) * D + g * kPerG);
#pragma unroll
    for (int i = 0; i < kPerG / 4; ++i) dst[i] = f32x4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
  }
  part[g][cl] = acc;
  __syncthreads();
  if (threadIdx.x < 32) {
    double sum = 0.0;
#pragma unroll
    for (int i = 0; i < kGroups; ++i) sum += part[i][threadIdx.x];
    const size_t slot = static_cast<size_t>(r) * n_ctiles + t;   // + term * n_rounds * n_ctiles
    const size_t term = static_cast<size_t>(n_rounds) * n_ctiles;
    max32_to(c < half ? norm_bits_up(sum) : 0u, bound_bits + kBoundCmax * term + slot);
    // the caller's near-tie total starts from zero (the fix-up kernel adds to it)
    if (threadIdx.x == 0 && t == 0 && r == 0 && n_near_ties != nullptr) *n_near_ties = 0;
    if (FRAG) {
      double sr = 0.0, sl = 0.0;
#pragma unroll
      for (int i = 0; i < kLoUnits; ++i) {
        sr += part_res[i][threadIdx.x];
        sl += part_lo[i][threadIdx.x];
      }
      max32_to(norm_bits_up(sr), bound_bits + kBoundRes * term + slot);
      max32_to(norm_bits_up(sl), bound_bits + kBoundLo * term + slot);
    }
  }
}

// One 16-byte piece per lane from global memory straight into LDS
// (global_load_lds): the wavefront writes 64 consecutive pieces starting at
// the wave-uniform address l.  The loads count against vmcnt; the workgroup
// barrier that follows them waits for that counter to drain.
__device__ __forceinline__ void lds_dma16(const u32x4* g, u32x4* l) {
#if __HIP_DEVICE_COMPILE__
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(l), 16, 0, 0);
#else
  (void)g;
  (void)l;
#endif
}

// --------------------------------------------------- MFMA hash (bf16) ----
typedef int i32x8 __attribute__((ext_vector_type(8)));

typedef float f32x16v __attribute__((ext_vector_type(16)));
typedef float f32x32v __attribute__((ext_vector_type(32)));
typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));

// 32 values (element 2i from even[i], 2i+1 from odd[i]) divided by the power
// of two `scale` and rounded to fp6 e2m3 codes, packed as 6-bit fields; and
// back.  The conversions write their results while still reading their
// sources, so the results are early-clobber outputs (never allocated over a
// source).
__device__ __forceinline__ u32x6 cvt_e2m3x32(f32x16v even, f32x16v odd, float scale) {
  u32x6 r;
  asm("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3\n\ts_nop 4" : "=&v"(r) : "v"(even), "v"(odd), "v"(scale));
  return r;
}

__device__ __forceinline__ f32x32v e2m3x32_to_f32(u32x6 p, float scale) {
  f32x32v r;
  asm("v_cvt_scalef32_pk32_f32_fp6 %0, %1, %2\n\ts_nop 4" : "=&v"(r) : "v"(p), "v"(scale));
  return r;
}

// v_mfma_scale_f32_32x32x64_f8f6f4 on fp6 e2m3 A and B (formats 2, 2); the B
// scale is byte `sel` of sb (sel is a constant once the caller's loops unroll).
__device__ __forceinline__ f32x16 mfma_fp6(i32x8 a, i32x8 b, f32x16 c, int sa, int sb, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 2, 0, sa, 0, sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 2, 0, sa, 1, sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 2, 0, sa, 2, sb);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 2, 0, sa, 3, sb);
  }
}

// fp6 B operand of one token for fp6 MFMA step kb: this lane (half g =
// lane/32) converts features k = 64kb + 32g + e, e = 0..31, into 6-bit field e,
// scaled by 2^-E with E per this block of 32 (its E8M0 byte 127 + E goes to
// *scale: each lane supplies its own block's scale).  Adds this lane's share
// of |x - x6|^2 to *err (float32 sum of exact differences: x has 8
// significant bits, x6 is x rounded to 4).
template <int D>
__device__ __forceinline__ i32x8 x_to_fp6(const uint16_t* __restrict__ xrow, bool live, int kb, int g, int* scale,
                                          float* err) {
  u32x4 raw[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    raw[h] = u32x4{0u, 0u, 0u, 0u};
    if (live) raw[h] = *reinterpret_cast<const u32x4*>(xrow + 64 * kb + 32 * g + 8 * h);
  }
  uint32_t mb = 0u;   // bf16 magnitudes order as integers
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) mb = max(mb, max(raw[h][e] & 0x7fffu, (raw[h][e] >> 16) & 0x7fffu));
  // scales stay normal floats; a block below 2^-124 then rounds to zero codes
  const int E = max(e2m3_block_exp(__uint_as_float(mb << 16)), -126);
  *scale = 127 + E;
  const float sc = ldexpf(1.0f, E);
  f32x16v even, odd;
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      even[4 * h + e] = __uint_as_float(raw[h][e] << 16);
      odd[4 * h + e] = __uint_as_float(raw[h][e] & 0xffff0000u);
    }
  const u32x6 w = cvt_e2m3x32(even, odd, sc);
  const f32x32v back = e2m3x32_to_f32(w, sc);
  float acc = *err;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float r0 = even[i] - back[2 * i], r1 = odd[i] - back[2 * i + 1];
    acc = fmaf(r0, r0, acc);
    acc = fmaf(r1, r1, acc);
  }
  *err = acc;
  return i32x8{static_cast<int>(w[0]), static_cast<int>(w[1]), static_cast<int>(w[2]),
               static_cast<int>(w[3]), static_cast<int>(w[4]), static_cast<int>(w[5]), 0, 0};
}

template <int D>
__global__ __launch_bounds__(kHashThreads, D == 128 ? 2 : 3) void hash_mfma_kernel(
    const uint16_t* __restrict__ qk, const u32x4* __restrict__ frag, const uint32_t* __restrict__ bound_bits,
    HashShape s, int32_t* __restrict__ buckets, NearTieList lst) {
  using FT = FragTile<D>;
  constexpr int kSteps = FT::kHiSteps;
  constexpr int kLoSteps = FT::kLoSteps;
  constexpr int kTileVec = FT::kVec;                 // 16-byte units per fragment tile
  constexpr int kChunks = kTileVec / 64;             // 1 KB wavefront copies per tile
  constexpr int kWaves = kHashThreads / 64;
  static_assert(kTileVec % 64 == 0, "tile copy works in 1 KB pieces");
  __shared__ u32x4 lds0[kTileVec];   // two separate buffers, so that the compiler can tell
  __shared__ u32x4 lds1[kTileVec];   // the copy into one from the reads of the other
  __shared__ int ntie;
  // Per-round maxima of the bound terms (float bits), gathered once here so
  // that the end of a round reads them from LDS instead of waiting on global
  // loads; with more rounds than fit, each round end reduces them itself.
  constexpr int kLdsRounds = 64;
  __shared__ uint32_t rbound[kLdsRounds][kBoundTerms];
  const bool rb_lds = s.n_rounds <= kLdsRounds;
  static_assert(kWaves * 32 * kStrips == kTokensPerBlock, "near-tie regions assume 256 tokens per block");
  if (threadIdx.x == 0) ntie = 0;
  lst.lds_count = &ntie;
  if (rb_lds) {
    for (int i = threadIdx.x; i < s.n_rounds * kBoundTerms; i += kHashThreads) (&rbound[0][0])[i] = 0u;
    __syncthreads();
    const int per_term = s.n_rounds * s.n_ctiles;
    for (int u = threadIdx.x; u < kBoundTerms * per_term; u += kHashThreads) {
      const int term = u / per_term, round = (u - term * per_term) / s.n_ctiles;
      atomicMax(&rbound[round][term], bound_bits[u]);   // non-negative float bits order as integers
    }
  }

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half_sel = lane >> 5;
  const int tok_base = (blockIdx.x * kWaves + wave) * (32 * kStrips);

  // B operands.  bf16: lane holds token (lane % 32), k = 16ks + 8*(lane/32) .. +7.
  // fp6: see x_to_fp6.  |x| and |x - x6| per token, rounded up.
  bf16x8 xf[kStrips][kSteps];
  i32x8 x6[kStrips][kLoSteps];
  static_assert(kStrips * kLoSteps <= 4, "fp6 scale bytes share one register");
  uint32_t xs6 = 0u;   // E8M0 byte of (st, kb) at byte st * kLoSteps + kb: the MFMA selects it
  // |x| and |x - x6| per strip, needed once per round: kept in LDS (read back
  // through a volatile pointer) rather than in registers the loop is short of.
  __shared__ float2 xnorm[kStrips][kHashThreads];
#pragma unroll
  for (int st = 0; st < kStrips; ++st) {
    const int tok = tok_base + 32 * st + (lane & 31);
    const bool live = tok < s.n_tokens;
    const uint16_t* xrow = qk + static_cast<size_t>(live ? tok : 0) * D;
    float acc = 0.0f;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (live) raw = *reinterpret_cast<const u32x4*>(xrow + 16 * ks + 8 * half_sel);
      xf[st][ks] = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float a = __uint_as_float(raw[e] << 16), b = __uint_as_float(raw[e] & 0xffff0000u);
        acc = fmaf(a, a, acc);
        acc = fmaf(b, b, acc);
      }
    }
    float err = 0.0f;
#pragma unroll
    for (int kb = 0; kb < kLoSteps; ++kb) {
      int sc;
      x6[st][kb] = x_to_fp6<D>(xrow, live, kb, half_sel, &sc, &err);
      xs6 |= static_cast<uint32_t>(sc) << (8 * (st * kLoSteps + kb));
    }
    acc += shfl_xor_f(acc, 32);
    err += shfl_xor_f(err, 32);
    // float32 sums of at most 256 squares: relative error below 2^-16
    xnorm[st][threadIdx.x] = make_float2(sqrtf(acc) * (1.0f + 1.0f / 65536.0f), sqrtf(err) * (1.0f + 1.0f / 65536.0f));
  }

  const int n_total = s.n_rounds * s.n_ctiles;
  // Prologue: tile 0 into buffer 0.
  for (int i = threadIdx.x; i < kTileVec; i += kHashThreads) lds0[i] = frag[i];
  __syncthreads();

  const uint32_t code_mask = (1u << s.code_bits) - 1u;
  const uint32_t keep_mask = 0x7fffffffu & ~code_mask;
  uint32_t k1[kStrips], k2[kStrips];
  int32_t smax[kStrips];
#pragma unroll
  for (int st = 0; st < kStrips; ++st) { k1[st] = 0u; k2[st] = 0u; smax[st] = INT32_MIN; }

  // Projections of tile n (lds buffer n & 1) into acc.
  auto mfma_tile = [&](f32x16 (&acc)[kStrips], const u32x4* cur) {
#pragma unroll
    for (int st = 0; st < kStrips; ++st)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[st][i] = 0.0f;
    // The small x.R_lo term first: the last writer of acc is then a bf16 MFMA,
    // whose result latency the key extraction that reads acc is scheduled for.
#pragma unroll
    for (int kb = 0; kb < kLoSteps; ++kb) {
      const u32x4 p0 = cur[FT::kHiVec + (2 * kb) * 64 + lane];
      const u32x4 p1 = cur[FT::kHiVec + (2 * kb + 1) * 64 + lane];
      const i32x8 a_lo = {static_cast<int>(p0[0]), static_cast<int>(p0[1]), static_cast<int>(p0[2]),
                          static_cast<int>(p0[3]), static_cast<int>(p1[0]), static_cast<int>(p1[1]), 0, 0};
      const int sa = static_cast<int>(p1[2]);
#pragma unroll
      for (int st = 0; st < kStrips; ++st)   // formats 2, 2: fp6 e2m3 A and B
        acc[st] = mfma_fp6(a_lo, x6[st][kb], acc[st], sa, static_cast<int>(xs6), st * kLoSteps + kb);
    }
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      const bf16x8 a_hi = __builtin_bit_cast(bf16x8, cur[ks * 64 + lane]);
#pragma unroll
      for (int st = 0; st < kStrips; ++st)
        acc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi, xf[st][ks], acc[st], 0, 0, 0);
    }
  };
  // Keys of tile n from acc: acc[i] is the projection on column
  // 32t + 8(i/4) + 4*half_sel + i%4.
  // Keys of the tile at column-tile index t of its round (tile n = round *
  // n_ctiles + t).
  auto keys_tile = [&](const f32x16 (&acc)[kStrips], int t) {
    const uint32_t tile_code = (static_cast<uint32_t>(t) << 5) | (static_cast<uint32_t>(half_sel) << 4);
#pragma unroll
    for (int st = 0; st < kStrips; ++st) {
      const uint32_t a1 = make_key(acc[st][0], keep_mask, 0u);
      const uint32_t a2 = make_key(acc[st][1], keep_mask, 1u);
      uint32_t t1 = max(a1, a2), t2 = min(a1, a2);
      int32_t sm = max(max(smax[st], __float_as_int(acc[st][0])), __float_as_int(acc[st][1]));
#pragma unroll
      for (int i = 2; i < 16; i += 2) {
        top2_push2(t1, t2, make_key(acc[st][i], keep_mask, static_cast<uint32_t>(i)),
                   make_key(acc[st][i + 1], keep_mask, static_cast<uint32_t>(i + 1)));
        sm = max(max(sm, __float_as_int(acc[st][i])), __float_as_int(acc[st][i + 1]));
      }
      smax[st] = sm;
      top2_merge(k1[st], k2[st], t1 | tile_code, t2 | tile_code);
    }
  };
  // After the last tile of a round: merge the two lanes that share each
  // token, decide, flag near-ties.
  auto round_end = [&](int t, int round) {
    if (t != s.n_ctiles - 1) return;
    float cmax, rho1, rho2;
    if (rb_lds) {
      cmax = __uint_as_float(rbound[round][kBoundCmax]);
      rho1 = __uint_as_float(rbound[round][kBoundRes]);
      rho2 = __uint_as_float(rbound[round][kBoundLo]);
    } else {
      cmax = round_bound(bound_bits, kBoundCmax, s.n_rounds, s.n_ctiles, round);
      rho1 = round_bound(bound_bits, kBoundRes, s.n_rounds, s.n_ctiles, round);
      rho2 = round_bound(bound_bits, kBoundLo, s.n_rounds, s.n_ctiles, round);
    }
#pragma unroll
    for (int st = 0; st < kStrips; ++st) {
      uint32_t o1 = shfl_xor_u(k1[st], 32), o2 = shfl_xor_u(k2[st], 32);
      top2_merge(k1[st], k2[st], o1, o2);
      const int32_t sm = max(smax[st], static_cast<int32_t>(shfl_xor_u(static_cast<uint32_t>(smax[st]), 32)));
      int tok = tok_base + 32 * st + lane;
      if (lane < 32 && tok < s.n_tokens) {
        const volatile float* xnv = reinterpret_cast<const volatile float*>(&xnorm[st][threadIdx.x]);
        const float2 xn = make_float2(xnv[0], xnv[1]);
        uint32_t c1 = k1[st] & code_mask, c2 = k2[st] & code_mask;
        auto col_of = [](uint32_t c) {
          uint32_t i = c & 15u, hs = (c >> 4) & 1u, tt = c >> 5;
          return static_cast<int>(32u * tt + 8u * (i >> 2) + 4u * hs + (i & 3u));
        };
        decide_and_store(k1[st], k2[st], sm, col_of(c1), col_of(c2),
                         split_gap_bound(xn.x, xn.y, cmax, rho1, rho2), s.code_bits, s.half, tok, s.seq_len,
                         s.n_rounds, round, buckets, lst);
      }
      k1[st] = 0u;
      k2[st] = 0u;
      smax[st] = INT32_MIN;
    }
  };
  // Tile n + 1 straight into the idle LDS buffer (global_load_lds): each
  // wavefront instruction fills 1 KB.  Issued before tile n's MFMAs, so the
  // copy overlaps them; the barrier at the end of the step waits for it.
  // After the last tile the copy repeats it (no branch).
  auto dma_next = [&](u32x4* dst, int n) {
    const u32x4* src = frag + static_cast<size_t>(min(n + 1, n_total - 1)) * kTileVec;
#pragma unroll
    for (int i = 0; i < (kChunks + kWaves - 1) / kWaves; ++i) {
      const int chunk = i * kWaves + wave;
      if (kChunks % kWaves == 0 || chunk < kChunks) lds_dma16(src + chunk * 64 + lane, dst + chunk * 64);
    }
  };

  // Software pipeline: the MFMAs of tile n are issued between the vector
  // instructions that turn tile n - 1's projections into keys (separate
  // accumulators, no dependence), so one wavefront keeps the matrix core and
  // the vector ALU busy at once.
  f32x16 acc_a[kStrips], acc_b[kStrips];
  int tp = 0, rp = 0;   // column tile and round of the tile whose keys the next step extracts
  auto step = [&](const u32x4* cur, u32x4* next, f32x16 (&acc)[kStrips], const f32x16 (&prev)[kStrips], int n) {
    dma_next(next, n);
    mfma_tile(acc, cur);
    keys_tile(prev, tp);
    // every LDS read of the tile's A operands first, so that none waits
    // behind the MFMAs; then one MFMA per five vector instructions
    __builtin_amdgcn_sched_group_barrier(0x100, kSteps + 2 * kLoSteps, 0);
#pragma unroll
    for (int i = 0; i < kStrips * (kSteps + kLoSteps); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // then five vector instructions
    }
    round_end(tp, rp);
    // advance (tp, rp) to tile n, with scalar increments instead of a division per step
    if (++tp == s.n_ctiles) {
      tp = 0;
      ++rp;
    }
    __syncthreads();   // also makes every wavefront's near-tie pushes visible to the count below
  };
  dma_next(lds1, 0);
  mfma_tile(acc_a, lds0);
  __syncthreads();
  int n = 1;
  for (; n + 1 < n_total; n += 2) {
    step(lds1, lds0, acc_b, acc_a, n);
    step(lds0, lds1, acc_a, acc_b, n + 1);
  }
  if (n < n_total) {   // n_total even: tile n (odd) is in lds1
    step(lds1, lds0, acc_b, acc_a, n);
    keys_tile(acc_b, tp);
  } else {
    keys_tile(acc_a, tp);
  }
  round_end(tp, rp);   // (tp, rp) is now the last tile's position
  __syncthreads();
  if (threadIdx.x == 0) lst.counts[blockIdx.x] = ntie;
}

// ------------------------------------------------- FMA hash (float32) ----
// One thread per token; rotation tiles of 64 columns staged in LDS.
template <int D>
__global__ __launch_bounds__(256) void hash_fma_kernel(const float* __restrict__ qk, const float* __restrict__ rot,
                                                       const uint32_t* __restrict__ cmax_bits, HashShape s,
                                                       int32_t* __restrict__ buckets, NearTieList lst) {
  constexpr int kCols = 64;
  __shared__ float rt[D][kCols];
  __shared__ int ntie;
  if (threadIdx.x == 0) ntie = 0;
  lst.lds_count = &ntie;
  const int tok = blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = tok < s.n_tokens;
  float x[D];
  float sq = 0.0f;
#pragma unroll
  for (int k = 0; k < D; ++k) {
    x[k] = live ? qk[static_cast<size_t>(tok) * D + k] : 0.0f;
    sq = fmaf(x[k], x[k], sq);
  }
  const float xnorm = sqrtf(sq) * 1.0000005f;
  const uint32_t code_mask = (1u << s.code_bits) - 1u;
  const uint32_t keep_mask = 0x7fffffffu & ~code_mask;
  for (int round = 0; round < s.n_rounds; ++round) {
    const float* R = rot + static_cast<size_t>(round) * D * s.half;
    uint32_t k1 = 0u, k2 = 0u;
    int32_t smax = INT32_MIN;
    for (int c0 = 0; c0 < s.half; c0 += kCols) {
      __syncthreads();
      for (int u = threadIdx.x; u < D * kCols; u += blockDim.x) {
        int k = u / kCols, j = u % kCols;
        rt[k][j] = (c0 + j < s.half) ? R[static_cast<size_t>(k) * s.half + c0 + j] : 0.0f;
      }
      __syncthreads();
      for (int j = 0; j < kCols && c0 + j < s.half; ++j) {
        float p = 0.0f;
#pragma unroll
        for (int k = 0; k < D; ++k) p = fmaf(x[k], rt[k][j], p);
        top2_push(k1, k2, make_key(p, keep_mask, static_cast<uint32_t>(c0 + j)));
        smax = max(smax, __float_as_int(p));
      }
    }
    const float cmax = round_bound(cmax_bits, kBoundCmax, s.n_rounds, s.n_ctiles, round);
    if (live) {
      int c1 = static_cast<int>(k1 & code_mask), c2 = static_cast<int>(k2 & code_mask);
      decide_and_store(k1, k2, smax, c1, c2, guard_tiny(kTauRel * xnorm * cmax, xnorm, cmax),
                       s.code_bits, s.half, tok, s.seq_len, s.n_rounds, round, buckets, lst);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) lst.counts[blockIdx.x] = ntie;
}

// ---------------------------------------------------------- fix-up ----
// Re-decide queued (token, round) pairs in float64 (products of a bf16 or
// float32 feature and a float32 rotation entry are exact in float64).  A group
// of 16 lanes takes one entry: for a pair, lane i holds features
// [i*D/16, (i+1)*D/16) and the two column dot products are summed across the
// group; for a full rescore, lane i scores columns i, i+16, ...
template <int D, bool BF16>
__global__ __launch_bounds__(256) void hash_fixup_kernel(const void* __restrict__ qk_raw, const float* __restrict__ rt,
                                                         HashShape s, int32_t* __restrict__ buckets,
                                                         const int32_t* __restrict__ counts, int n_regions, int cap,
                                                         const int32_t* __restrict__ entries_all, int32_t* n_near_ties) {
  constexpr int kPer = D / 16;
  constexpr int kGroups = 256 / 16;
  const int sub = threadIdx.x & 15;
  const int group = threadIdx.x >> 4;
  int seen = 0;
  for (int region = blockIdx.x; region < n_regions; region += gridDim.x) {
    const int count = counts[region];
    seen += count;
    const int32_t* entries = entries_all + 3 * static_cast<size_t>(region) * cap;
    for (int e = group; e < count; e += kGroups) {
      const int tok = entries[3 * static_cast<size_t>(e)];
      const int w1 = entries[3 * static_cast<size_t>(e) + 1];
      const int w2 = entries[3 * static_cast<size_t>(e) + 2];
      const int round = w1 & 0x7fffffff;
      const bool full = (w1 & static_cast<int>(0x80000000u)) != 0;
      const float* R = rt + static_cast<size_t>(round) * s.half * D;
      auto xval = [&](int k) -> double {
        if (BF16) return static_cast<double>(bf16_to_f32(static_cast<const uint16_t*>(qk_raw)[static_cast<size_t>(tok) * D + k]));
        return static_cast<double>(static_cast<const float*>(qk_raw)[static_cast<size_t>(tok) * D + k]);
      };
      // Best candidate as (value, bucket): larger value wins, equal values go to the lower bucket.
      double best_v = -1.0;
      int best_b = 0x7fffffff;
      auto offer = [&](double p, int c) {
        double v = p >= 0.0 ? p : -p;
        int b = p >= 0.0 ? c : c + s.half;   // p == 0: +p (lower bucket) and -p tie; lower wins
        if (v > best_v || (v == best_v && b < best_b)) { best_v = v; best_b = b; }
      };
      if (!full) {
        const int c1 = w2 & 0xffff, c2 = (w2 >> 16) & 0xffff;
        double xv[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) xv[i] = xval(sub * kPer + i);
        double p1 = 0.0, p2 = 0.0;
        const f32x4* r1 = reinterpret_cast<const f32x4*>(R + static_cast<size_t>(min(c1, s.half - 1)) * D + sub * kPer);
        const f32x4* r2 = reinterpret_cast<const f32x4*>(R + static_cast<size_t>(min(c2, s.half - 1)) * D + sub * kPer);
#pragma unroll
        for (int i = 0; i < kPer / 4; ++i) {
          const f32x4 a = r1[i], b = r2[i];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            p1 += xv[4 * i + j] * static_cast<double>(a[j]);
            p2 += xv[4 * i + j] * static_cast<double>(b[j]);
          }
        }
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) {
          p1 += shfl_xor_d(p1, off);
          p2 += shfl_xor_d(p2, off);
        }
        if (c1 < s.half) offer(p1, c1);
        if (c2 < s.half && c2 != c1) offer(p2, c2);
      } else {
        for (int c = sub; c < s.half; c += 16) {
          const f32x4* rc = reinterpret_cast<const f32x4*>(R + static_cast<size_t>(c) * D);
          double p = 0.0;
#pragma unroll 2
          for (int i = 0; i < D / 4; ++i) {
            const f32x4 a = rc[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) p += xval(4 * i + j) * static_cast<double>(a[j]);
          }
          offer(p, c);
        }
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) {
          double ov = shfl_xor_d(best_v, off);
          int ob = __shfl_xor(best_b, off, 64);
          if (ov > best_v || (ov == best_v && ob < best_b)) { best_v = ov; best_b = ob; }
        }
      }
      if (sub == 0) {
        int bh = tok / s.seq_len, pos = tok - bh * s.seq_len;
        buckets[(static_cast<size_t>(bh) * s.n_rounds + round) * s.seq_len + pos] = best_b;
      }
    }
  }
  if (n_near_ties != nullptr && threadIdx.x == 0 && seen > 0) atomicAdd(n_near_ties, seen);
}

__global__ void fill_zero_kernel(int32_t* p, size_t n) {
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (; i < n; i += stride) p[i] = 0;
}

int ceil_log2(int v) {
  int b = 0;
  while ((1 << b) < v) ++b;
  return b;
}

}  // namespace

HashShape make_hash_shape(int batch, int heads, int seq_len, int d, int n_rounds, int n_buckets) {
  HashShape s{};
  s.n_tokens = batch * heads * seq_len;
  s.seq_len = seq_len;
  s.d = d;
  s.n_rounds = n_rounds;
  s.n_buckets = n_buckets;
  s.half = n_buckets / 2;
  s.n_ctiles = (s.half + 31) / 32;
  // MFMA codes: 4 bits value index, 1 bit lane half, then the tile index.
  s.code_bits = std::max(5 + ceil_log2(s.n_ctiles), ceil_log2(std::max(s.half, 2)));
  return s;
}

HashScratch hash_scratch(const HashShape& s) {
  HashScratch h{};
  // per tile: bf16 R_hi (2 bytes) and fp6 R_lo with its scales (1 byte) for 32 columns x d
  h.frag_bytes = align_up(static_cast<size_t>(s.n_rounds) * s.n_ctiles * 32 * s.d * 3, 256);
  h.rt_bytes = align_up(static_cast<size_t>(s.n_rounds) * s.half * s.d * sizeof(float), 256);
  // per-tile column-norm maxima [kBoundTerms][n_rounds][n_ctiles]
  h.bound_bytes = align_up(static_cast<size_t>(s.n_rounds) * s.n_ctiles * kBoundTerms * sizeof(uint32_t), 256);
  const size_t regions = (static_cast<size_t>(s.n_tokens) + kTokensPerBlock - 1) / kTokensPerBlock;
  h.counter_bytes = align_up(regions * sizeof(int32_t), 256);
  h.list_bytes = align_up(regions * kTokensPerBlock * s.n_rounds * 3 * sizeof(int32_t), 256);
  h.total = h.frag_bytes + h.rt_bytes + h.bound_bytes + h.counter_bytes + h.list_bytes;
  return h;
}

hipError_t launch_fill_zero_buckets(int32_t* buckets, size_t n, hipStream_t stream) {
  unsigned grid = static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 4096));
  if (grid == 0) grid = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, stream, buckets, n);
  return hipGetLastError();
}

hipError_t launch_hash(const void* qk, bool bf16, const float* rotations, const HashShape& s, int32_t* buckets,
                       int32_t* n_near_ties, void* workspace, hipStream_t stream, hipEvent_t* marks) {
  HashScratch h = hash_scratch(s);
  char* ws = static_cast<char*>(workspace);
  u32x4* frag = reinterpret_cast<u32x4*>(ws);
  ws += h.frag_bytes;
  float* rt = reinterpret_cast<float*>(ws);
  ws += h.rt_bytes;
  uint32_t* bound = reinterpret_cast<uint32_t*>(ws);                          // [kBoundTerms][n_rounds][n_ctiles]
  ws += h.bound_bytes;
  int32_t* counts = reinterpret_cast<int32_t*>(ws);
  ws += h.counter_bytes;
  int32_t* list = reinterpret_cast<int32_t*>(ws);
  const int n_regions = (s.n_tokens + kTokensPerBlock - 1) / kTokensPerBlock;
  const int cap = kTokensPerBlock * s.n_rounds;
  NearTieList lst{counts, list, cap, nullptr};

  const dim3 pg(s.n_ctiles, s.n_rounds);
  const dim3 grid(n_regions);
  if (bf16) {
    const uint16_t* x = static_cast<const uint16_t*>(qk);
    if (s.d == 64) {
      hipLaunchKernelGGL((hash_prepare_kernel<64, true>), pg, dim3(256), 0, stream, rotations, s.half, s.n_rounds, s.n_ctiles, frag, rt, bound, n_near_ties);
      if (marks) (void)hipEventRecord(marks[0], stream);
      hipLaunchKernelGGL(hash_mfma_kernel<64>, grid, dim3(kHashThreads), 0, stream, x, frag, bound, s, buckets, lst);
    } else {
      hipLaunchKernelGGL((hash_prepare_kernel<128, true>), pg, dim3(256), 0, stream, rotations, s.half, s.n_rounds, s.n_ctiles, frag, rt, bound, n_near_ties);
      if (marks) (void)hipEventRecord(marks[0], stream);
      hipLaunchKernelGGL(hash_mfma_kernel<128>, grid, dim3(kHashThreads), 0, stream, x, frag, bound, s, buckets, lst);
    }
  } else {
    const float* x = static_cast<const float*>(qk);
    if (s.d == 64) {
      hipLaunchKernelGGL((hash_prepare_kernel<64, false>), pg, dim3(256), 0, stream, rotations, s.half, s.n_rounds, s.n_ctiles, frag, rt, bound, n_near_ties);
      if (marks) (void)hipEventRecord(marks[0], stream);
      hipLaunchKernelGGL(hash_fma_kernel<64>, grid, dim3(256), 0, stream, x, rotations, bound, s, buckets, lst);
    } else {
      hipLaunchKernelGGL((hash_prepare_kernel<128, false>), pg, dim3(256), 0, stream, rotations, s.half, s.n_rounds, s.n_ctiles, frag, rt, bound, n_near_ties);
      if (marks) (void)hipEventRecord(marks[0], stream);
      hipLaunchKernelGGL(hash_fma_kernel<128>, grid, dim3(256), 0, stream, x, rotations, bound, s, buckets, lst);
    }
  }
  if (marks) (void)hipEventRecord(marks[1], stream);
  const int fix_blocks = std::min(n_regions, 2048);
  if (s.d == 64) {
    if (bf16)
      hipLaunchKernelGGL((hash_fixup_kernel<64, true>), dim3(fix_blocks), dim3(256), 0, stream, qk, rt, s, buckets, counts, n_regions, cap, list, n_near_ties);
    else
      hipLaunchKernelGGL((hash_fixup_kernel<64, false>), dim3(fix_blocks), dim3(256), 0, stream, qk, rt, s, buckets, counts, n_regions, cap, list, n_near_ties);
  } else {
    if (bf16)
      hipLaunchKernelGGL((hash_fixup_kernel<128, true>), dim3(fix_blocks), dim3(256), 0, stream, qk, rt, s, buckets, counts, n_regions, cap, list, n_near_ties);
    else
      hipLaunchKernelGGL((hash_fixup_kernel<128, false>), dim3(fix_blocks), dim3(256), 0, stream, qk, rt, s, buckets, counts, n_regions, cap, list, n_near_ties);
  }
  if (marks) (void)hipEventRecord(marks[2], stream);
  return hipGetLastError();
}

}  // namespace rlsh
