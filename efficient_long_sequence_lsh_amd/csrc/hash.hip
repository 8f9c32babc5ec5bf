// Stage 1: LSH bucket ids, h(x) = argmax([xR; -xR]).
//
// "Reformer: The Efficient Transformer" (research summary), Key points, LSH
// attention bullet: each vector is hashed as the argmax of the concatenation
// of its rotation xR and the negation -xR.  Bucket k < b/2 is +(xR)_k and
// bucket b/2 + k is -(xR)_k; ties go to the lowest bucket index.
//
// Design for gfx950
//   * The projection x.R is a dense contraction (tokens x d) . (d x b/2), so
//     bf16 inputs run on MFMA (v_mfma_f32_32x32x16_bf16).  Float32 accuracy is
//     kept by splitting R = R_hi + R_lo into two bfloat16 terms: bf16 x bf16
//     products are exact in float32, and the split leaves a residual below
//     2^-16 |R|.  Float32 inputs use a plain FMA kernel.
//   * The matrix product is computed transposed, D = R^T X^T, so that each lane
//     receives 16 projections of ONE token per 32x32 tile.  Every projection is
//     turned into an ordered 32-bit key: the float's magnitude bits shifted up
//     by one, its sign in bit 0 and a candidate code in the low mantissa bits.
//     A running top-two of keys per lane costs one med3 and one max per value;
//     the two lanes sharing a token merge once per round.
//   * The top-two keys give the two leading candidates and their gap.  When the
//     gap is below a bound on the float32 error (Cauchy-Schwarz:
//     |x|_2 * max_j |R_j|_2 scaled by 2^-12, plus the key truncation), the
//     (position, round) is queued and a fix-up kernel re-decides it in float64
//     between those two candidates (or over all columns when even the leading
//     magnitude is within the bound, e.g. x = 0).
//   * Rotation fragments are pre-arranged in global memory in the exact order
//     the MFMA A operand wants them, so the cooperative copy into LDS is a
//     straight coalesced memcpy and every wave reads 1 KB contiguous per
//     fragment (no bank conflicts).  Tiles are double-buffered through LDS.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>

namespace rlsh {

namespace {

constexpr float kTauRel = 1.0f / 4096.0f;   // 2^-12 of |x|_2 * max_j |R_j|_2
constexpr int kHashThreads = 256;           // 4 wavefronts
constexpr int kStrips = 2;                  // 32-token strips per wavefront

// --------------------------------------------------------------- keys ----
// key = [magnitude bits 30..0 of the float, shifted up by one] [sign in bit 0],
// with bits 1..code_bits replaced by a candidate code.  Unsigned order of keys
// is the order of |p| truncated to (23 - code_bits) mantissa bits.
__device__ __forceinline__ uint32_t rotl1(uint32_t b) { return __builtin_amdgcn_alignbit(b, b, 31); }

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
  return __uint_as_float(((key & ~code_mask) & ~1u) >> 1);
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
__device__ __forceinline__ void decide_and_store(uint32_t k1, uint32_t k2, int col1, int col2, float xnorm,
                                                 float cmax, int code_bits, int half, int tok, int seq_len,
                                                 int n_rounds, int round, int32_t* buckets, NearTieList lst) {
  const uint32_t code_mask = ((1u << code_bits) - 1u) << 1;
  float m1 = key_magnitude(k1, code_mask);
  float m2 = key_magnitude(k2, code_mask);
  float tau = kTauRel * xnorm * cmax + m1 * __uint_as_float((127u + code_bits - 22u) << 23);
  int bucket = col1 + ((k1 & 1u) ? half : 0);
  int bh = tok / seq_len, pos = tok - bh * seq_len;
  buckets[(static_cast<size_t>(bh) * n_rounds + round) * seq_len + pos] = bucket;
  bool full = !(m1 > tau);
  if (full || (m1 - m2) <= tau) push_near_tie(lst, tok, round, full, col1, col2);
}

// ------------------------------------------------------ preparation ----
// Zero the per-round column-norm maxima and the caller's near-tie total.
__global__ void hash_init_kernel(uint32_t* cmax_bits, int n_rounds, int32_t* n_near_ties) {
  for (int t = threadIdx.x; t < n_rounds; t += blockDim.x) cmax_bits[t] = 0u;
  if (threadIdx.x == 0 && n_near_ties != nullptr) *n_near_ties = 0;
}

// Per-call set-up, one workgroup per (tile of 32 rotation columns, round):
//  - (FRAG) split-bf16 fragments of R in MFMA A-operand order: fragment
//    (round r, tile t, k-step ks, term, lane l) holds, for column
//    c = 32t + l%32 and k0 = 16ks + 8(l/32), the 8 values R[r][k0 + e][c]
//    (zero for c >= half) as bf16 hi (term 0) or lo = bf16(R - hi) (term 1);
//  - R transposed to float32 [round][column][k], so that the fix-up reads a
//    column as one contiguous row;
//  - column norms (float64 sums, rounded up) folded into a per-round max.
template <int D, bool FRAG>
__global__ __launch_bounds__(256) void hash_prepare_kernel(const float* __restrict__ rot, int half, int n_ctiles,
                                                           u32x4* __restrict__ frag, float* __restrict__ rt,
                                                           uint32_t* __restrict__ cmax_bits) {
  constexpr int kSteps = D / 16;
  constexpr int kGroups = 8;               // k-ranges per column
  constexpr int kPerG = D / kGroups;       // 8 or 16 values
  __shared__ double part[kGroups][32];
  const int t = blockIdx.x, r = blockIdx.y;
  const float* R = rot + static_cast<size_t>(r) * D * half;
  if (FRAG) {
    for (int u = threadIdx.x; u < kSteps * 64; u += blockDim.x) {
      const int ks = u / 64, l = u % 64;
      const int c = 32 * t + (l & 31);
      const int k0 = 16 * ks + 8 * (l >> 5);
      u32x4 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float v0 = 0.0f, v1 = 0.0f;
        if (c < half) {
          v0 = R[static_cast<size_t>(k0 + e) * half + c];
          v1 = R[static_cast<size_t>(k0 + e + 1) * half + c];
        }
        const uint16_t h0 = f32_to_bf16_rne(v0), h1 = f32_to_bf16_rne(v1);
        const uint16_t l0 = f32_to_bf16_rne(v0 - bf16_to_f32(h0)), l1 = f32_to_bf16_rne(v1 - bf16_to_f32(h1));
        hi[e / 2] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
        lo[e / 2] = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
      }
      const size_t base = (((static_cast<size_t>(r) * n_ctiles + t) * kSteps + ks) * 2) * 64 + l;
      frag[base] = hi;
      frag[base + 64] = lo;
    }
  }
  const int cl = threadIdx.x & 31, g = threadIdx.x >> 5;
  const int c = 32 * t + cl;
  double acc = 0.0;
  if (c < half) {
    float v[kPerG];
#pragma unroll
    for (int i = 0; i < kPerG; ++i) {
      v[i] = R[static_cast<size_t>(g * kPerG + i) * half + c];
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
    uint32_t bits = 0u;
    if (c < half) bits = __float_as_uint(static_cast<float>(sqrt(sum)) * 1.0000005f);   // round up slightly
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) bits = max(bits, static_cast<uint32_t>(__shfl_xor(static_cast<int>(bits), off, 32)));
    if (threadIdx.x == 0) atomicMax(cmax_bits + r, bits);
  }
}

// One 16-byte piece per lane from global memory straight into LDS
// (global_load_lds): the wavefront writes 64 consecutive pieces starting at
// the wave-uniform address l.  The loads count against vmcnt; the workgroup
// barrier that follows them waits for that counter to drain.
__device__ __forceinline__ void lds_dma16(const u32x4* g, u32x4* l) {
#if __HIP_DEVICE_COMPILE__
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(l), 16, 0, 0);
#endif
}

// --------------------------------------------------- MFMA hash (bf16) ----
template <int D>
__global__ __launch_bounds__(kHashThreads, 4) void hash_mfma_kernel(
    const uint16_t* __restrict__ qk, const u32x4* __restrict__ frag, const uint32_t* __restrict__ cmax_bits,
    HashShape s, int32_t* __restrict__ buckets, NearTieList lst) {
  constexpr int kSteps = D / 16;
  constexpr int kTileVec = kSteps * 2 * 64;                   // 16-byte units per fragment tile
  constexpr int kPerThread = kTileVec / kHashThreads;
  static_assert(kTileVec % kHashThreads == 0, "tile copy must divide evenly");
  __shared__ u32x4 lds[2][kTileVec];
  __shared__ int ntie;
  static_assert(kHashThreads / 64 * 32 * kStrips == kTokensPerBlock, "near-tie regions assume 256 tokens per block");
  if (threadIdx.x == 0) ntie = 0;
  lst.lds_count = &ntie;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half_sel = lane >> 5;
  const int tok_base = (blockIdx.x * (kHashThreads / 64) + wave) * (32 * kStrips);

  // X^T operand (B): lane holds token (lane % 32), k = 16ks + 8*(lane/32) .. +7.
  bf16x8 xf[kStrips][kSteps];
  float xsq[kStrips];
#pragma unroll
  for (int st = 0; st < kStrips; ++st) {
    int tok = tok_base + 32 * st + (lane & 31);
    float acc = 0.0f;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (tok < s.n_tokens)
        raw = *reinterpret_cast<const u32x4*>(qk + static_cast<size_t>(tok) * D + 16 * ks + 8 * half_sel);
      xf[st][ks] = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float a = __uint_as_float(raw[e] << 16), b = __uint_as_float(raw[e] & 0xffff0000u);
        acc = fmaf(a, a, acc);
        acc = fmaf(b, b, acc);
      }
    }
    acc += shfl_xor_f(acc, 32);
    xsq[st] = sqrtf(acc) * 1.0000005f;
  }

  const int n_total = s.n_rounds * s.n_ctiles;
  // Prologue: tile 0 into buffer 0.
  {
    const u32x4* src = frag;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) lds[0][threadIdx.x + i * kHashThreads] = src[threadIdx.x + i * kHashThreads];
  }
  __syncthreads();

  const uint32_t code_mask = ((1u << s.code_bits) - 1u) << 1;
  const uint32_t keep_mask = ~code_mask;
  uint32_t k1[kStrips], k2[kStrips];
#pragma unroll
  for (int st = 0; st < kStrips; ++st) { k1[st] = 0u; k2[st] = 0u; }

  for (int n = 0; n < n_total; ++n) {
    const int buf = n & 1;
    const int round = n / s.n_ctiles;
    const int t = n - round * s.n_ctiles;
    const bool has_next = (n + 1) < n_total;

    f32x16 acc[kStrips];
#pragma unroll
    for (int st = 0; st < kStrips; ++st)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[st][i] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      bf16x8 a_hi = __builtin_bit_cast(bf16x8, lds[buf][(ks * 2 + 0) * 64 + lane]);
      bf16x8 a_lo = __builtin_bit_cast(bf16x8, lds[buf][(ks * 2 + 1) * 64 + lane]);
#pragma unroll
      for (int st = 0; st < kStrips; ++st) {
        acc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi, xf[st][ks], acc[st], 0, 0, 0);
        acc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_lo, xf[st][ks], acc[st], 0, 0, 0);
      }
    }
    // Next tile straight into the other LDS buffer (global_load_lds): each
    // wavefront instruction fills 1 KB; the barrier below waits for it.
    if (has_next) {
      const u32x4* src = frag + static_cast<size_t>(n + 1) * kTileVec;
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) {
        const int chunk = i * (kHashThreads / 64) + wave;
        lds_dma16(src + chunk * 64 + lane, &lds[buf ^ 1][chunk * 64]);
      }
    }

    // Keys: acc[i] is the projection on column 32t + 8(i/4) + 4*half_sel + i%4.
    const uint32_t tile_code = (static_cast<uint32_t>(t) << 5) | (static_cast<uint32_t>(half_sel) << 4);
#pragma unroll
    for (int st = 0; st < kStrips; ++st) {
      uint32_t a1 = (rotl1(__float_as_uint(acc[st][0])) & keep_mask) | (0u << 1);
      uint32_t a2 = (rotl1(__float_as_uint(acc[st][1])) & keep_mask) | (1u << 1);
      uint32_t t1 = max(a1, a2), t2 = min(a1, a2);
#pragma unroll
      for (int i = 2; i < 16; ++i) {
        uint32_t key = (rotl1(__float_as_uint(acc[st][i])) & keep_mask) | (static_cast<uint32_t>(i) << 1);
        top2_push(t1, t2, key);
      }
      top2_merge(k1[st], k2[st], t1 | (tile_code << 1), t2 | (tile_code << 1));
    }

    if (t == s.n_ctiles - 1) {
      // End of a round: merge the two lanes that share each token, decide, flag.
      const float cmax = __uint_as_float(cmax_bits[round]);
#pragma unroll
      for (int st = 0; st < kStrips; ++st) {
        uint32_t o1 = shfl_xor_u(k1[st], 32), o2 = shfl_xor_u(k2[st], 32);
        top2_merge(k1[st], k2[st], o1, o2);
        int tok = tok_base + 32 * st + lane;
        if (lane < 32 && tok < s.n_tokens) {
          uint32_t c1 = (k1[st] & code_mask) >> 1, c2 = (k2[st] & code_mask) >> 1;
          auto col_of = [](uint32_t c) {
            uint32_t i = c & 15u, hs = (c >> 4) & 1u, tt = c >> 5;
            return static_cast<int>(32u * tt + 8u * (i >> 2) + 4u * hs + (i & 3u));
          };
          decide_and_store(k1[st], k2[st], col_of(c1), col_of(c2), xsq[st], cmax, s.code_bits, s.half, tok,
                           s.seq_len, s.n_rounds, round, buckets, lst);
        }
        k1[st] = 0u;
        k2[st] = 0u;
      }
    }

    __syncthreads();
  }
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
  const uint32_t code_mask = ((1u << s.code_bits) - 1u) << 1;
  for (int round = 0; round < s.n_rounds; ++round) {
    const float* R = rot + static_cast<size_t>(round) * D * s.half;
    uint32_t k1 = 0u, k2 = 0u;
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
        uint32_t key = (rotl1(__float_as_uint(p)) & ~code_mask) | (static_cast<uint32_t>(c0 + j) << 1);
        top2_push(k1, k2, key);
      }
    }
    if (live) {
      int c1 = static_cast<int>((k1 & code_mask) >> 1), c2 = static_cast<int>((k2 & code_mask) >> 1);
      decide_and_store(k1, k2, c1, c2, xnorm, __uint_as_float(cmax_bits[round]), s.code_bits, s.half, tok,
                       s.seq_len, s.n_rounds, round, buckets, lst);
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
  h.frag_bytes = align_up(static_cast<size_t>(s.n_rounds) * s.n_ctiles * 32 * s.d * 2 * sizeof(uint16_t), 256);
  h.rt_bytes = align_up(static_cast<size_t>(s.n_rounds) * s.half * s.d * sizeof(float), 256);
  h.cmax_bytes = align_up(static_cast<size_t>(s.n_rounds) * sizeof(uint32_t), 256);
  const size_t regions = (static_cast<size_t>(s.n_tokens) + kTokensPerBlock - 1) / kTokensPerBlock;
  h.counter_bytes = align_up(regions * sizeof(int32_t), 256);
  h.list_bytes = align_up(regions * kTokensPerBlock * s.n_rounds * 3 * sizeof(int32_t), 256);
  h.total = h.frag_bytes + h.rt_bytes + h.cmax_bytes + h.counter_bytes + h.list_bytes;
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
  uint32_t* cmax = reinterpret_cast<uint32_t*>(ws);
  ws += h.cmax_bytes;
  int32_t* counts = reinterpret_cast<int32_t*>(ws);
  ws += h.counter_bytes;
  int32_t* list = reinterpret_cast<int32_t*>(ws);
  const int n_regions = (s.n_tokens + kTokensPerBlock - 1) / kTokensPerBlock;
  const int cap = kTokensPerBlock * s.n_rounds;
  NearTieList lst{counts, list, cap, nullptr};

  hipLaunchKernelGGL(hash_init_kernel, dim3(1), dim3(256), 0, stream, cmax, s.n_rounds, n_near_ties);
  const dim3 pg(s.n_ctiles, s.n_rounds);
  const dim3 grid(n_regions);
  if (bf16) {
    const uint16_t* x = static_cast<const uint16_t*>(qk);
    if (s.d == 64) {
      hipLaunchKernelGGL((hash_prepare_kernel<64, true>), pg, dim3(256), 0, stream, rotations, s.half, s.n_ctiles, frag, rt, cmax);
      if (marks) (void)hipEventRecord(marks[0], stream);
      hipLaunchKernelGGL(hash_mfma_kernel<64>, grid, dim3(kHashThreads), 0, stream, x, frag, cmax, s, buckets, lst);
    } else {
      hipLaunchKernelGGL((hash_prepare_kernel<128, true>), pg, dim3(256), 0, stream, rotations, s.half, s.n_ctiles, frag, rt, cmax);
      if (marks) (void)hipEventRecord(marks[0], stream);
      hipLaunchKernelGGL(hash_mfma_kernel<128>, grid, dim3(kHashThreads), 0, stream, x, frag, cmax, s, buckets, lst);
    }
  } else {
    const float* x = static_cast<const float*>(qk);
    if (s.d == 64) {
      hipLaunchKernelGGL((hash_prepare_kernel<64, false>), pg, dim3(256), 0, stream, rotations, s.half, s.n_ctiles, frag, rt, cmax);
      if (marks) (void)hipEventRecord(marks[0], stream);
      hipLaunchKernelGGL(hash_fma_kernel<64>, grid, dim3(256), 0, stream, x, rotations, cmax, s, buckets, lst);
    } else {
      hipLaunchKernelGGL((hash_prepare_kernel<128, false>), pg, dim3(256), 0, stream, rotations, s.half, s.n_ctiles, frag, rt, cmax);
      if (marks) (void)hipEventRecord(marks[0], stream);
      hipLaunchKernelGGL(hash_fma_kernel<128>, grid, dim3(256), 0, stream, x, rotations, cmax, s, buckets, lst);
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
