// Stages 3 + 4: gather sorted rows and run chunked attention for every round.
//
// "Reformer: The Efficient Transformer" (research summary), Key points:
//   LSH attention bullet -- the sorted positions form chunks of m whose queries
//   see the keys of their own chunk and of the preceding one;
//   Shared-QK bullet -- queries and keys are the same vectors, and a position's
//   own key is excluded unless nothing else is left for it (that fallback is
//   applied when the rounds are combined).
// Readings where the page is silent: score x_i.x_j / sqrt(d); chunk 0 has no
// predecessor; optional causal mask by original position (key j < query i);
// every key of the window is eligible.
//
// Output per round and position: z = log sum exp(s) over the valid keys and
// o = softmax-weighted average of their v rows (o = 0, z = -inf if none),
// written by ORIGINAL position, so the un-sort is done by this store and the
// round combine becomes a pure streaming pass.
//
// Design for gfx950
//   * One workgroup = 4 wavefronts = a tile of 64 consecutive sorted slots
//     (16 queries per wavefront); it walks a run of consecutive query tiles so
//     the chunk loaded as "own" for one tile is still in L2 (same XCD) when the
//     next tile reads it as "previous".
//   * Keys are visited in tiles of 64 sorted slots gathered through perm
//     straight into LDS (rows are 128 / 256 contiguous bytes: coalesced).
//   * Scores are computed transposed, S^T = K Q^T, with the 16x16x32 bf16 MFMA
//     (16x16x4 f32 for float32 inputs): each lane then owns one query and 4
//     keys per 16-key block, which is exactly the B-operand layout that the
//     P.V product O^T = V^T P^T needs, so probabilities never leave registers.
//     V is stored transposed in LDS for the bf16 A operand.
//   * Online softmax in the log2 domain with wavefront-level row max
//     (2 lane shuffles per key tile); row sums are reduced once at the end.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>
#include <cmath>
#include <type_traits>

namespace rlsh {

namespace {

constexpr int kQTile = 64;       // sorted slots per query tile (4 waves x 16)
constexpr int kKTile = 64;       // sorted slots per key tile
constexpr int kRunTiles = 4;     // query tiles per workgroup on grids that fill the chip

struct AttnShape {
  int seq_len;
  int chunk;       // m' = min(chunk_len, seq_len)
  int n_rounds;
  int n_qt;        // query tiles per segment
  int causal;
  float scale_log2;  // log2(e) / sqrt(d)
};

template <int D, bool BF16>
struct AttnLds;

template <int D>
struct alignas(16) AttnLds<D, true> {
  static constexpr int kKPitch = D + 8;      // bf16 elements per K row (16-byte pad)
  static constexpr int kVPitch = kKTile + 4; // bf16 elements per transposed V row
  uint16_t k[kKTile * kKPitch];
  uint16_t vt[D * kVPitch];
  int kpos[kKTile];
};

template <int D>
struct alignas(16) AttnLds<D, false> {
  static constexpr int kKPitch = D + 4;      // floats per K row
  static constexpr int kVPitch = D + 4;      // floats per V row (row-major)
  float k[kKTile * kKPitch];
  float v[kKTile * kVPitch];
  int kpos[kKTile];
};

template <int D, bool BF16>
__global__ __launch_bounds__(256) void chunk_attend_kernel(const void* __restrict__ qk_raw,
                                                           const void* __restrict__ v_raw,
                                                           const int32_t* __restrict__ perm_all, AttnShape s,
                                                           int run_tiles, float* __restrict__ o_rounds,
                                                           float* __restrict__ z_rounds) {
  using Lds = AttnLds<D, BF16>;
  __shared__ Lds sh;

  const int seg = blockIdx.y;                    // (batch*head)*n_rounds + round
  const int bh = seg / s.n_rounds;
  const int L = s.seq_len;
  const int m = s.chunk;
  const int32_t* perm = perm_all + static_cast<size_t>(seg) * L;
  const size_t row0 = static_cast<size_t>(bh) * L;   // first row of this (batch, head) in qk / v

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q16 = lane & 15;      // query column owned by this lane
  const int g = lane >> 4;        // 4-lane group index

  const int qt_begin = blockIdx.x * run_tiles;
  const int qt_end = min(s.n_qt, qt_begin + run_tiles);

  for (int qt = qt_begin; qt < qt_end; ++qt) {
    const int s0 = qt * kQTile;
    const int qslot = s0 + 16 * wave + q16;
    const bool qlive = qslot < L;
    const int qpos = qlive ? perm[qslot] : -1;
    const int cq = qlive ? qslot / m : 0;
    const int wlo = max(0, (cq - 1) * m);
    const int whi = qlive ? min(L, (cq + 1) * m) : 0;
    const int c_lo = s0 / m;
    const int c_hi = min(s0 + kQTile - 1, L - 1) / m;
    const int ks_begin = max(0, (c_lo - 1) * m);
    const int ks_end = min(L, (c_hi + 1) * m);

    // Query fragments (B operand of S^T = K Q^T).
    constexpr int kQF = BF16 ? D / 32 : D / 4;
    using QFrag = typename std::conditional<BF16, bf16x8, float>::type;
    QFrag qf[kQF];
    if constexpr (BF16) {
      const uint16_t* qk = static_cast<const uint16_t*>(qk_raw);
#pragma unroll
      for (int kk = 0; kk < kQF; ++kk) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (qlive) raw = *reinterpret_cast<const u32x4*>(qk + (row0 + qpos) * D + 32 * kk + 8 * g);
        qf[kk] = __builtin_bit_cast(bf16x8, raw);
      }
    } else {
      const float* qk = static_cast<const float*>(qk_raw);
#pragma unroll
      for (int kk = 0; kk < kQF; ++kk) qf[kk] = qlive ? qk[(row0 + qpos) * D + 4 * kk + g] : 0.0f;
    }

    float m_run = -INFINITY;
    float l_run = 0.0f;
    f32x4 oacc[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int kt0 = ks_begin; kt0 < ks_end; kt0 += kKTile) {
      __syncthreads();   // previous readers of the LDS tile are done
      // ---- gather 64 key rows (qk and v) through perm into LDS ----
      if constexpr (BF16) {
        const uint16_t* qk = static_cast<const uint16_t*>(qk_raw);
        const uint16_t* vv = static_cast<const uint16_t*>(v_raw);
        constexpr int kChunks = D / 8;                 // 16-byte pieces per row
        for (int u = threadIdx.x; u < kKTile * kChunks; u += 256) {
          const int row = u / kChunks, ch = u % kChunks;
          const int slot = kt0 + row;
          u32x4 kr = {0u, 0u, 0u, 0u}, vr = {0u, 0u, 0u, 0u};
          if (slot < ks_end) {
            const size_t prow = row0 + perm[slot];
            kr = *reinterpret_cast<const u32x4*>(qk + prow * D + 8 * ch);
            vr = *reinterpret_cast<const u32x4*>(vv + prow * D + 8 * ch);
          }
          *reinterpret_cast<u32x4*>(&sh.k[row * Lds::kKPitch + 8 * ch]) = kr;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sh.vt[(8 * ch + 2 * e) * Lds::kVPitch + row] = static_cast<uint16_t>(vr[e] & 0xffffu);
            sh.vt[(8 * ch + 2 * e + 1) * Lds::kVPitch + row] = static_cast<uint16_t>(vr[e] >> 16);
          }
        }
      } else {
        const float* qk = static_cast<const float*>(qk_raw);
        const float* vv = static_cast<const float*>(v_raw);
        constexpr int kChunks = D / 4;
        for (int u = threadIdx.x; u < kKTile * kChunks; u += 256) {
          const int row = u / kChunks, ch = u % kChunks;
          const int slot = kt0 + row;
          f32x4 kr = {0.0f, 0.0f, 0.0f, 0.0f}, vr = {0.0f, 0.0f, 0.0f, 0.0f};
          if (slot < ks_end) {
            const size_t prow = row0 + perm[slot];
            kr = *reinterpret_cast<const f32x4*>(qk + prow * D + 4 * ch);
            vr = *reinterpret_cast<const f32x4*>(vv + prow * D + 4 * ch);
          }
          *reinterpret_cast<f32x4*>(&sh.k[row * Lds::kKPitch + 4 * ch]) = kr;
          *reinterpret_cast<f32x4*>(&sh.v[row * Lds::kVPitch + 4 * ch]) = vr;
        }
      }
      if (threadIdx.x < kKTile) {
        const int slot = kt0 + threadIdx.x;
        sh.kpos[threadIdx.x] = slot < ks_end ? perm[slot] : -1;
      }
      __syncthreads();

      // ---- S^T = K Q^T: lane holds S[q16][16t + 4g + j] ----
      f32x4 sc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (BF16) {
#pragma unroll
          for (int kk = 0; kk < kQF; ++kk) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(&sh.k[(16 * t + q16) * Lds::kKPitch + 32 * kk + 8 * g]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), qf[kk], acc, 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < kQF; ++kk) {
            const float a = sh.k[(16 * t + q16) * Lds::kKPitch + 4 * kk + g];
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, qf[kk], acc, 0, 0, 0);
          }
        }
        sc[t] = acc;
      }

      // ---- masks, scale, tile max ----
      float tmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kr = 16 * t + 4 * g + j;
          const int ksl = kt0 + kr;
          const int kp = sh.kpos[kr];
          bool ok = (ksl >= wlo) && (ksl < whi) && (ksl != qslot);
          if (s.causal) ok = ok && (kp < qpos);
          const float val = ok ? sc[t][j] * s.scale_log2 : -INFINITY;
          sc[t][j] = val;
          tmax = fmaxf(tmax, val);
        }
      tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
      tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);     // 0 when m_run = -inf
      float psum = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = __builtin_amdgcn_exp2f(sc[t][j] - m_use);   // exp2(-inf) = 0 for masked keys
          sc[t][j] = p;
          psum += p;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) oacc[dt][j] *= alpha;

      // ---- O^T += V^T P^T ----
      if constexpr (BF16) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          u32x4 pb;
          pb[0] = pack_bf16x2(sc[2 * kb][0], sc[2 * kb][1]);
          pb[1] = pack_bf16x2(sc[2 * kb][2], sc[2 * kb][3]);
          pb[2] = pack_bf16x2(sc[2 * kb + 1][0], sc[2 * kb + 1][1]);
          pb[3] = pack_bf16x2(sc[2 * kb + 1][2], sc[2 * kb + 1][3]);
          const bf16x8 bop = __builtin_bit_cast(bf16x8, pb);
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) {
            const uint16_t* vrow = &sh.vt[(16 * dt + q16) * Lds::kVPitch + 32 * kb + 4 * g];
            u32x4 a;
            const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16);
            a[0] = lo[0];
            a[1] = lo[1];
            a[2] = hi[0];
            a[3] = hi[1];
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), bop, oacc[dt], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int kr = 16 * t + 4 * g + j;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
              const float a = sh.v[kr * Lds::kVPitch + 16 * dt + q16];
              oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sc[t][j], oacc[dt], 0, 0, 0);
            }
          }
      }
    }

    // ---- finish: row sums across the 4 lane groups, normalise, store ----
    float lsum = l_run;
    lsum += shfl_xor_f(lsum, 16);
    lsum += shfl_xor_f(lsum, 32);
    if (qlive) {
      const bool empty = (m_run == -INFINITY) || !(lsum > 0.0f);
      const float inv = empty ? 0.0f : 1.0f / lsum;
      const size_t orow = static_cast<size_t>(seg) * L + qpos;
      float* op = o_rounds + orow * D;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        f32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = oacc[dt][j] * inv;
        *reinterpret_cast<f32x4*>(op + 16 * dt + 4 * g) = r;
      }
      if (g == 0) z_rounds[orow] = empty ? -INFINITY : (m_run + log2f(lsum)) * 0.69314718055994531f;
    }
  }
}

// ---------------------------------------------------------------------------
// Chunks of exactly 64 slots (one key tile per chunk), bf16 inputs.
//
// A workgroup walks a run of consecutive chunks of one segment.  LDS holds two
// chunks (K rows and transposed V): the previous chunk and the current one, so
// every chunk is gathered from HBM once per run.  While chunk c is computed,
// chunk c+1 is gathered into registers and written into the buffer of chunk
// c-1 afterwards.  Query fragments come from the current chunk in LDS (the
// queries of a chunk are its own keys).  The whole 128-key window of a query
// fits in registers, so the softmax is single pass.  Runs are mapped to blocks
// so that neighbouring runs share an XCD (and its L2) for the one chunk two
// runs both read.
constexpr int kRun64 = 16;  // chunks per workgroup at most

// Chunks per run.  Longer runs gather fewer previous chunks twice; at d = 64
// with short segments, runs of 8 measured faster (the 12K image shape: 0.877
// against 0.895 ms per forward; 64K text with d = 128: 0.824 against 0.832 ms
// the other way; 512K tokens: no difference).
int run_chunks(int d, int seq_len) { return d == 64 && seq_len <= 32768 ? 8 : kRun64; }

// K and V rows are both kept row-major.  K rows are padded by 16 bytes (the
// S^T A-operand reads of 16 rows x 16 bytes hit distinct banks); V rows by 32
// bytes so that the transposing reads below (16 rows x 32 bytes per
// instruction) and the 16-byte row writes are both conflict-free.
template <int D>
struct alignas(16) Lds64 {
  static constexpr int kKPitch = D + 8;
  static constexpr int kVPitch = D + 16;
  uint16_t k[2][kKTile * kKPitch];
  uint16_t v[2][kKTile * kVPitch];
  int pos[(kRun64 + 1) * kKTile];   // perm of the run's chunks (and the one before)
};

template <int D>
struct TileRegs {
  static constexpr int kChunks = D / 8;                  // 16-byte pieces per row
  static constexpr int kPer = kKTile * kChunks / 256;    // pieces per thread
  u32x4 k[kPer];
  u32x4 v[kPer];
};

// Rows of one chunk straight from HBM into registers; positions come from LDS.
template <int D>
__device__ __forceinline__ void gather_tile(TileRegs<D>& t, const uint16_t* __restrict__ qk,
                                            const uint16_t* __restrict__ vv, const int* pos, size_t row0) {
  constexpr int kChunks = TileRegs<D>::kChunks;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kPer; ++i) {
    const int u = threadIdx.x + 256 * i;
    const int row = u / kChunks, ch = u % kChunks;
    const size_t prow = row0 + pos[row];
    t.k[i] = *reinterpret_cast<const u32x4*>(qk + prow * D + 8 * ch);
    t.v[i] = *reinterpret_cast<const u32x4*>(vv + prow * D + 8 * ch);
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& t, Lds64<D>& sh, int buf) {
  constexpr int kChunks = TileRegs<D>::kChunks;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kPer; ++i) {
    const int u = threadIdx.x + 256 * i;
    const int row = u / kChunks, ch = u % kChunks;
    *reinterpret_cast<u32x4*>(&sh.k[buf][row * Lds64<D>::kKPitch + 8 * ch]) = t.k[i];
    *reinterpret_cast<u32x4*>(&sh.v[buf][row * Lds64<D>::kVPitch + 8 * ch]) = t.v[i];
  }
}

// Where a round's per-position results go.
//  kSinkF32:     o float32 [.., d] and z float32 (the stage entry point).
//  kSinkCompact: o as a compact row (CompactRow: float16 at d = 64, 12-bit
//                block floating point at d = 128) that carries its own z and
//                scale exponent, so a round's record at a position is exactly
//                its row.
//  kSinkFinal:   the last round of the bf16 pipeline combines in place: it
//                reads the compact results of the earlier rounds at the
//                query's position, applies the logsumexp weights (self
//                fallback when no round has a target) and writes the bf16
//                output row, so its own o is never stored.
//  kSinkFinal + 1 + np: the same with the np earlier rounds' rows loaded at
//                the start of each chunk, so their latency hides behind the
//                chunk's own work (np = r - 1 for the common round counts).
constexpr int kSinkF32 = 0;
constexpr int kSinkCompact = 1;
constexpr int kSinkFinal = 2;
constexpr int sink_final_prefetch(int np) { return kSinkFinal + 1 + np; }

struct RoundSink {
  float* o;              // kSinkF32
  float* z;              // kSinkF32
  uint16_t* o16;         // kSinkCompact: this launch's rounds; kSinkFinal: earlier rounds (read)
  const uint16_t* v;     // kSinkFinal: self fallback rows
  uint16_t* out;         // kSinkFinal: output [bh, L, d]
  float* lse;            // kSinkFinal, optional: log of the combined normaliser per position
};

// Compact rows.  A row is held by the four lanes q16 + 16g (g = 0..3); lane g
// has the D/4 values of features 16dt + 4g + j (dt < D/16, j < 4), value
// i = 4dt + j of the lane.  Two encodings:
//   d = 64, float16: value i is the float16 of o * 2^-k, k = max(e - 14, -116)
//     for the row's largest magnitude in [2^e, 2^(e+1)) (so it lands in
//     [2^14, 2^15) and neither overflows nor falls into subnormals), two to a
//     dword at the feature's own place in the row (128 bytes);
//   d = 128, 12-bit block floating point: value i is the integer
//     q = rne(o * 2^-E) in [-2048, 2047], with E = max(e - 10, -116) for the
//     row's largest magnitude in [2^e, 2^(e+1)); the lane's 32 integers are
//     packed at bits 12i of 12 dwords stored at byte 48g of the row (192
//     bytes, three 64-byte sectors instead of the four of float16).
//     Absolute error at most 2^(E-1) <= 2^-11 of the row's largest magnitude.
// Either way lanes g = 0, 1 and 2 carry 16-bit pieces of the row's metadata in
// the lowest bit of their first 16 values (bit i of the piece in value i):
// the low and high halves of z's float bits and the scale exponent (k or E)
// plus 128.  So a round's record at a position is exactly its row, and no
// separate 8-byte entry has its sector fetched whole by the last round's
// gather.  The bit replaced costs at most one more unit in the last place
// (float16: 2^-10 of the value; 12-bit: 2^E) in 48 of the row's values.
template <int D>
struct CompactRow {
  static constexpr bool kBfp = D == 128;
  static constexpr int kBytes = kBfp ? 3 * D / 2 : 2 * D;   // per row
  static constexpr int kWords = kBfp ? 12 : D / 8;            // dwords per lane
};

// The lane's dwords of a stored row.
template <int D>
__device__ __forceinline__ void load_row_words(const uint16_t* o16, size_t row, int g,
                                               uint32_t (&w)[CompactRow<D>::kWords]) {
  const unsigned char* base = reinterpret_cast<const unsigned char*>(o16) + row * CompactRow<D>::kBytes;
  if constexpr (CompactRow<D>::kBfp) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(base + 48 * g + 16 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) w[4 * i + e] = v[e];
    }
  } else {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(base + 2 * (16 * dt + 4 * g));
      w[2 * dt] = v[0];
      w[2 * dt + 1] = v[1];
    }
  }
}

// The metadata piece a lane carries (the lowest bits of its first 16 values).
template <int D>
__device__ __forceinline__ uint32_t row_meta_piece(const uint32_t (&w)[CompactRow<D>::kWords]) {
  uint32_t p = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int bit = CompactRow<D>::kBfp ? 12 * i : 16 * i;
    p |= ((w[bit >> 5] >> (bit & 31)) & 1u) << i;
  }
  return p;
}

// (z, scale exponent) of the row whose pieces the four lanes of query row
// q16 hold; every lane of the wavefront must take part.
__device__ __forceinline__ float2 row_meta(uint32_t piece, int q16) {
  const uint32_t lo = static_cast<uint32_t>(__shfl(static_cast<int>(piece), q16, 64));
  const uint32_t hi = static_cast<uint32_t>(__shfl(static_cast<int>(piece), q16 + 16, 64));
  const uint32_t ex = static_cast<uint32_t>(__shfl(static_cast<int>(piece), q16 + 32, 64));
  return make_float2(__uint_as_float((lo & 0xffffu) | (hi << 16)), static_cast<float>(static_cast<int>(ex & 0xffu) - 128));
}

// Value i of the lane's stored row, without its scale.
template <int D>
__device__ __forceinline__ float row_value(const uint32_t (&w)[CompactRow<D>::kWords], int i) {
  if constexpr (CompactRow<D>::kBfp) {
    const int bit = 12 * i, k = bit >> 5, off = bit & 31;
    const uint32_t x = off <= 20 ? w[k] >> off : __builtin_amdgcn_alignbit(w[k + 1], w[k], off);
    return static_cast<float>(static_cast<int32_t>(x << 20) >> 20);   // sign-extend the low 12 bits
  } else {
    const uint32_t x = w[i >> 1];
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>((i & 1) ? x >> 16 : x & 0xffffu)));
  }
}

// Encodes this lane's part of a row: o = oacc * inv, z, and writes it.
// amax is the row's largest |o| (over all four lanes).
template <int D>
__device__ __forceinline__ void store_compact_row(uint16_t* o16, size_t row, int g, const f32x4 (&oacc)[D / 16],
                                                  float inv, float amax, float zval) {
  const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xffu) - 127;
  int ex;
  float f;
  if constexpr (CompactRow<D>::kBfp) {
    ex = max(e - 10, -116);
    f = __uint_as_float(static_cast<uint32_t>(127 - ex) << 23) * inv;   // 2^-E / lsum
  } else {
    ex = max(e - 14, -116);   // k: amax * 2^-k in [2^14, 2^15), tiny rows scaled up
    f = __uint_as_float(static_cast<uint32_t>(127 - ex) << 23) * inv;
  }
  const uint32_t zb = __float_as_uint(zval);
  const uint32_t piece = g == 0 ? (zb & 0xffffu) : g == 1 ? (zb >> 16) : static_cast<uint32_t>(ex + 128);
  const uint32_t keep = g < 3 ? ~1u : ~0u;
  auto meta_bit = [&](int i) -> uint32_t { return (g < 3 && i < 16) ? (piece >> i) & 1u : 0u; };
  unsigned char* base = reinterpret_cast<unsigned char*>(o16) + row * CompactRow<D>::kBytes;
  if constexpr (CompactRow<D>::kBfp) {
    uint32_t w[12];
#pragma unroll
    for (int k = 0; k < 12; ++k) w[k] = 0u;
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      const int q = min(max(static_cast<int>(rintf(oacc[i >> 2][i & 3] * f)), -2048), 2047);
      uint32_t u = static_cast<uint32_t>(q) & 0xfffu;
      if (i < 16) u = (u & keep) | meta_bit(i);
      const int bit = 12 * i, k = bit >> 5, off = bit & 31;
      w[k] |= u << off;
      if (off > 20) w[k + 1] |= u >> (32 - off);
    }
#pragma unroll
    for (int i = 0; i < 3; ++i)
      *reinterpret_cast<u32x4*>(base + 48 * g + 16 * i) = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
  } else {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      uint32_t h[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[j] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(oacc[dt][j] * f));
        if (4 * dt + j < 16) h[j] = (h[j] & keep) | meta_bit(4 * dt + j);
      }
      *reinterpret_cast<u32x2*>(base + 2 * (16 * dt + 4 * g)) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    }
  }
}

// One chunk: queries = rows of buffer `cur`, keys = rows of `prv` (previous
// chunk, if any) and `cur`.  Writes o and z by original position.
template <int D, int MODE>
__device__ __forceinline__ void attend_chunk64(const Lds64<D>& sh, int cur, int prv, bool has_prev, const int* cpos,
                                               const int* ppos, int causal, float scale_log2, size_t orow_base,
                                               size_t row0, int seq_len, int n_prev, RoundSink out) {
  constexpr int kKP = Lds64<D>::kKPitch;
  constexpr int kVP = Lds64<D>::kVPitch;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q16 = lane & 15;
  const int g = lane >> 4;
  const int qrow = 16 * wave + q16;          // query row inside the chunk
  const int qpos = cpos[qrow];
  // Final-round sink with a compile-time round count: this lane's features
  // of the earlier rounds' o rows (which carry their (z, k)), loaded now.
  constexpr bool kPre = MODE > kSinkFinal;
  constexpr int kNP = kPre ? MODE - kSinkFinal - 1 : 0;
  constexpr int kNPA = kNP > 0 ? kNP : 1;
  uint32_t opre[kNPA][CompactRow<D>::kWords];
  if constexpr (kPre) {
    const size_t prow0 = row0 * (kNP + 1) + qpos;
#pragma unroll
    for (int rho = 0; rho < kNP; ++rho) load_row_words<D>(out.o16, prow0 + static_cast<size_t>(rho) * seq_len, g, opre[rho]);
  }
  bf16x8 qf[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sh.k[cur][qrow * kKP + 32 * kk + 8 * g]));

  // S^T for 8 subtiles of 16 keys: 0..3 previous chunk, 4..7 own chunk.
  f32x4 sc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int buf = t < 4 ? prv : cur;
    const int kr0 = 16 * (t & 3);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (t >= 4 || has_prev) {
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&sh.k[buf][(kr0 + q16) * kKP + 32 * kk + 8 * g]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), qf[kk], acc, 0, 0, 0);
      }
    }
    sc[t] = acc;
  }
  // Masks on the raw scores (the scale is applied inside the exponent):
  // no previous chunk -> its subtiles are empty; the query's own key (row
  // qrow) sits in subtile 4 + wave at element q16 - 4g; causal -> key
  // position must precede the query position.
  if (!has_prev) {
#pragma unroll
    for (int t = 0; t < 4; ++t) sc[t] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  }
  const int jd = q16 - 4 * g;   // diagonal element index when 0 <= jd < 4
#pragma unroll
  for (int t = 4; t < 8; ++t)
    if (t - 4 == wave) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j == jd) sc[t][j] = -INFINITY;
    }
  if (causal) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int* kp = t < 4 ? ppos : cpos;
      const u32x4 kp4 = *reinterpret_cast<const u32x4*>(kp + 16 * (t & 3) + 4 * g);   // positions of this lane's 4 keys
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[t][j] = static_cast<int>(kp4[j]) < qpos ? sc[t][j] : -INFINITY;
    }
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int t = 0; t < 8; ++t) tmax = fmaxf(tmax, fmaxf(fmaxf(sc[t][0], sc[t][1]), fmaxf(sc[t][2], sc[t][3])));
  tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
  tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
  // p = 2^((s - max) * scale); a row with no valid key keeps every p = 0.
  const float m_off = (tmax == -INFINITY) ? 0.0f : -tmax * scale_log2;
  float psum = 0.0f;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sc[t][j], scale_log2, m_off));
      sc[t][j] = p;
      psum += p;
    }

  f32x4 oacc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    if (kb < 2 && !has_prev) continue;
    const int buf = kb < 2 ? prv : cur;
    const int kb_in = kb & 1;
    u32x4 pb;
    pb[0] = pack_bf16x2(sc[2 * kb][0], sc[2 * kb][1]);
    pb[1] = pack_bf16x2(sc[2 * kb][2], sc[2 * kb][3]);
    pb[2] = pack_bf16x2(sc[2 * kb + 1][0], sc[2 * kb + 1][1]);
    pb[3] = pack_bf16x2(sc[2 * kb + 1][2], sc[2 * kb + 1][3]);
    const bf16x8 bop = __builtin_bit_cast(bf16x8, pb);
    // A operand (V^T, 16 features x 32 keys): lane 16g+i needs feature i of
    // keys 32kb + 4g + {0..3} (first half) and 32kb + 16 + 4g + {0..3}
    // (second half); lane 16g + 4k + q points at key row (.. + k), features
    // 16dt + 4q .. +3, and the transposing read hands each lane its column.
    const uint16_t* vbase = &sh.v[buf][(32 * kb_in + 4 * g + (q16 >> 2)) * kVP + 4 * (q16 & 3)];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const u32x2 lo = lds_read_tr16(vbase + 16 * dt);
      const u32x2 hi = lds_read_tr16(vbase + 16 * kVP + 16 * dt);
      u32x4 a;
      a[0] = lo[0];
      a[1] = lo[1];
      a[2] = hi[0];
      a[3] = hi[1];
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), bop, oacc[dt], 0, 0, 0);
    }
  }
  float lsum = psum;
  lsum += shfl_xor_f(lsum, 16);
  lsum += shfl_xor_f(lsum, 32);
  const bool empty = (tmax == -INFINITY) || !(lsum > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / lsum;
  const size_t orow = orow_base + qpos;
  const float zval = empty ? -INFINITY : (tmax * scale_log2 + log2f(lsum)) * 0.69314718055994531f;
  if constexpr (MODE == kSinkF32) {
    float* op = out.o + orow * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      f32x4 r;
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = oacc[dt][j] * inv;
      *reinterpret_cast<f32x4*>(op + 16 * dt + 4 * g) = r;
    }
    if (g == 0) out.z[orow] = zval;
  } else if constexpr (MODE == kSinkCompact) {
    // Row maximum (the row is spread over the 4 lanes q16 + 16g).
    float amax = 0.0f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(oacc[dt][j]));
    amax = fmaxf(amax, shfl_xor_f(amax, 16));
    amax = fmaxf(amax, shfl_xor_f(amax, 32));
    store_compact_row<D>(out.o16, orow, g, oacc, inv, amax * inv, zval);
  } else {
    // Round combine at this position: rounds 0..n_prev-1 are stored compact
    // at rows (round0 + rho) * L + qpos; this round's o is still in registers.
    const int np = kPre ? kNP : n_prev;
    const size_t prow0 = row0 * (np + 1) + qpos;   // round 0 of this (batch, head)
    // (z, k) of round rho's row: from the prefetched features, or (uncommon
    // round counts) from the first four steps of the row, read here and again
    // with the rest of the row when it is added.
    auto row_meta_of = [&](int rho) -> float2 {
      if constexpr (kPre) return row_meta(row_meta_piece<D>(opre[rho]), q16);
      uint32_t w[CompactRow<D>::kWords];
      load_row_words<D>(out.o16, prow0 + static_cast<size_t>(rho) * seq_len, g, w);
      return row_meta(row_meta_piece<D>(w), q16);
    };
    float2 zpre[kNPA];
    float zmax = zval;
    if constexpr (kPre) {
#pragma unroll
      for (int rho = 0; rho < kNP; ++rho) {
        zpre[rho] = row_meta_of(rho);
        zmax = fmaxf(zmax, zpre[rho].x);
      }
    } else {
      for (int rho = 0; rho < np; ++rho) zmax = fmaxf(zmax, row_meta_of(rho).x);
    }
    u32x2 res[D / 16];
    float row_lse = -INFINITY;
    if (zmax == -INFINITY) {   // no round has a valid target: the token's own value
      const uint16_t* vp = out.v + (row0 + qpos) * D;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) res[dt] = *reinterpret_cast<const u32x2*>(vp + 16 * dt + 4 * g);
    } else {
      const float w_this = empty ? 0.0f : __expf(zval - zmax);
      float wsum = w_this;
      const float c_this = w_this * inv;
      float acc[D / 16][4];
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[dt][j] = oacc[dt][j] * c_this;
      // Adds round rho's stored row (values times 2^exponent) with its weight.
      auto add_round = [&](const float2 e, const uint32_t (&w)[CompactRow<D>::kWords]) {
        const float wt = __expf(e.x - zmax);   // 0 for rounds without a target
        wsum += wt;
        const float ws = wt * __uint_as_float(static_cast<uint32_t>(127 + static_cast<int>(e.y)) << 23);   // wt * 2^ex
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[dt][j] = fmaf(ws, row_value<D>(w, 4 * dt + j), acc[dt][j]);
      };
      if constexpr (kPre) {
#pragma unroll
        for (int rho = 0; rho < kNP; ++rho) add_round(zpre[rho], opre[rho]);
      } else {
        for (int rho = 0; rho < np; ++rho) {
          uint32_t w[CompactRow<D>::kWords];
          load_row_words<D>(out.o16, prow0 + static_cast<size_t>(rho) * seq_len, g, w);
          add_round(row_meta(row_meta_piece<D>(w), q16), w);
        }
      }
      const float rs = 1.0f / wsum;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        res[dt][0] = pack_bf16x2(acc[dt][0] * rs, acc[dt][1] * rs);
        res[dt][1] = pack_bf16x2(acc[dt][2] * rs, acc[dt][3] * rs);
      }
      row_lse = zmax + __logf(wsum);
    }
    if (out.lse != nullptr && g == 0) out.lse[row0 + qpos] = row_lse;
    uint16_t* dst = out.out + (row0 + qpos) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<u32x2*>(dst + 16 * dt + 4 * g) = res[dt];
  }
}

template <int D, int MODE>
__global__ __launch_bounds__(256, 2) void chunk_attend64_kernel(const uint16_t* __restrict__ qk,
                                                                const uint16_t* __restrict__ vv,
                                                                const int32_t* __restrict__ perm_all, AttnShape s,
                                                                int n_seg, int launch_rounds, int round_base,
                                                                int runs_per_seg, int run_len, int per_xcd,
                                                                RoundSink out) {
  __shared__ Lds64<D> sh;
  // XCD-aware mapping: hardware places block b on XCD b % 8; give each XCD a
  // contiguous range of runs.
  const int b = blockIdx.x;
  const int logical = (b % 8) * per_xcd + b / 8;
  if (logical >= n_seg * runs_per_seg) return;
  const int lseg = logical / runs_per_seg;
  const int run = logical - lseg * runs_per_seg;
  const int bh = lseg / launch_rounds;
  const int seg = bh * s.n_rounds + round_base + (lseg - bh * launch_rounds);
  const int L = s.seq_len;
  const int32_t* perm = perm_all + static_cast<size_t>(seg) * L;
  const size_t row0 = static_cast<size_t>(bh) * L;
  const size_t orow_base = static_cast<size_t>(seg) * L;
  const int n_prev = s.n_rounds - 1;   // used by kSinkFinal (the last round)
  const int c_begin = run * run_len;
  const int c_end = min(s.n_qt, c_begin + run_len);

  // Positions of the run's chunks: pos[(c - c_begin + 1) * 64 + row] = perm[c * 64 + row].
  {
    const int s_lo = (c_begin - 1) * kKTile;
    const int s_hi = c_end * kKTile;
    for (int i = threadIdx.x; i < (run_len + 1) * kKTile; i += 256) {
      const int slot = s_lo + i;
      sh.pos[i] = (slot >= 0 && slot < s_hi) ? perm[slot] : 0;
    }
  }
  __syncthreads();
  auto pos_of = [&](int c) -> const int* { return &sh.pos[(c - c_begin + 1) * kKTile]; };

  // Register ping-pong: while chunk c is computed, chunk c+1 is already in
  // registers (or landing) and chunk c+2 is being gathered.
  TileRegs<D> ra, rb;
  if (c_begin > 0) gather_tile<D>(rb, qk, vv, pos_of(c_begin - 1), row0);
  gather_tile<D>(ra, qk, vv, pos_of(c_begin), row0);
  if (c_begin > 0) store_tile<D>(rb, sh, 1);          // previous chunk lives in buffer 1
  store_tile<D>(ra, sh, 0);
  if (c_begin + 1 < c_end) gather_tile<D>(ra, qk, vv, pos_of(c_begin + 1), row0);
  __syncthreads();

  int cur = 0;
  int c = c_begin;
  while (true) {
    // ra holds chunk c+1 (if any)
    if (c + 2 < c_end) gather_tile<D>(rb, qk, vv, pos_of(c + 2), row0);
    attend_chunk64<D, MODE>(sh, cur, cur ^ 1, c > 0, pos_of(c), pos_of(c - 1), s.causal, s.scale_log2, orow_base,
                            row0, L, n_prev, out);
    __syncthreads();
    if (c + 1 < c_end) store_tile<D>(ra, sh, cur ^ 1);
    __syncthreads();
    cur ^= 1;
    if (++c >= c_end) break;
    // rb holds chunk c+1 (if any)
    if (c + 2 < c_end) gather_tile<D>(ra, qk, vv, pos_of(c + 2), row0);
    attend_chunk64<D, MODE>(sh, cur, cur ^ 1, c > 0, pos_of(c), pos_of(c - 1), s.causal, s.scale_log2, orow_base,
                            row0, L, n_prev, out);
    __syncthreads();
    if (c + 1 < c_end) store_tile<D>(rb, sh, cur ^ 1);
    __syncthreads();
    cur ^= 1;
    if (++c >= c_end) break;
  }
}

template <int D, int MODE>
hipError_t launch_fast64(const void* qk, const void* v, const int32_t* perm, int bh, int launch_rounds, int round_base,
                         AttnShape s, RoundSink out, hipStream_t stream) {
  const int run_len = std::min(kRun64, std::max(1, run_chunks(D, s.seq_len)));
  const int runs_per_seg = (s.n_qt + run_len - 1) / run_len;
  const int n_seg = bh * launch_rounds;
  const int total = n_seg * runs_per_seg;
  if (total == 0) return hipSuccess;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL((chunk_attend64_kernel<D, MODE>), dim3(8 * per_xcd), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(qk), static_cast<const uint16_t*>(v), perm, s, n_seg, launch_rounds,
                     round_base, runs_per_seg, run_len, per_xcd, out);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_typed(const void* qk, const void* v, const int32_t* perm, int n_seg, AttnShape s, float* o, float* z,
                        hipStream_t stream) {
  // Each query tile gathers its own key tiles, so a workgroup per tile costs
  // nothing in reuse: small grids take one tile per workgroup to spread over
  // more CUs (1024 positions, one head: 16 workgroups instead of 4).
  const long long grid4 = static_cast<long long>((s.n_qt + kRunTiles - 1) / kRunTiles) * n_seg;
  const int run = grid4 >= 512 ? kRunTiles : 1;
  dim3 grid((s.n_qt + run - 1) / run, n_seg);
  hipLaunchKernelGGL((chunk_attend_kernel<D, BF16>), grid, dim3(256), 0, stream, qk, v, perm, s, run, o, z);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_attend(const void* qk, const void* v, bool bf16, const int32_t* perm, int bh, int seq_len,
                               int d, int n_rounds, int chunk_len, bool causal, float* o_rounds, float* z_rounds,
                               hipStream_t stream) {
  AttnShape s{};
  s.seq_len = seq_len;
  s.chunk = std::min(chunk_len, seq_len);
  s.n_rounds = n_rounds;
  s.n_qt = (seq_len + kQTile - 1) / kQTile;
  s.causal = causal ? 1 : 0;
  s.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(d)));
  const int n_seg = bh * n_rounds;
  if (bf16 && s.chunk == kKTile && seq_len % kKTile == 0) {
    RoundSink out{o_rounds, z_rounds, nullptr, nullptr, nullptr, nullptr};
    return d == 64 ? launch_fast64<64, kSinkF32>(qk, v, perm, bh, n_rounds, 0, s, out, stream)
                   : launch_fast64<128, kSinkF32>(qk, v, perm, bh, n_rounds, 0, s, out, stream);
  }
  if (d == 64) {
    return bf16 ? launch_typed<64, true>(qk, v, perm, n_seg, s, o_rounds, z_rounds, stream)
                : launch_typed<64, false>(qk, v, perm, n_seg, s, o_rounds, z_rounds, stream);
  }
  return bf16 ? launch_typed<128, true>(qk, v, perm, n_seg, s, o_rounds, z_rounds, stream)
              : launch_typed<128, false>(qk, v, perm, n_seg, s, o_rounds, z_rounds, stream);
}

bool compact_rounds_supported(bool bf16, int seq_len, int chunk_len) {
  return bf16 && std::min(chunk_len, seq_len) == kKTile && seq_len % kKTile == 0;
}

template <int MODE>
hipError_t launch_final(const void* qk, const void* v, const int32_t* perm, int bh, int d, AttnShape s, RoundSink sink,
                        hipStream_t stream) {
  return d == 64 ? launch_fast64<64, MODE>(qk, v, perm, bh, 1, s.n_rounds - 1, s, sink, stream)
                 : launch_fast64<128, MODE>(qk, v, perm, bh, 1, s.n_rounds - 1, s, sink, stream);
}

hipError_t launch_attend_combine_compact(const void* qk, const void* v, const int32_t* perm, int bh, int seq_len,
                                         int d, int n_rounds, bool causal, uint16_t* o16, void* out,
                                         float* lse, hipStream_t stream, hipEvent_t* mark) {
  AttnShape s{};
  s.seq_len = seq_len;
  s.chunk = kKTile;
  s.n_rounds = n_rounds;
  s.n_qt = seq_len / kKTile;
  s.causal = causal ? 1 : 0;
  s.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(d)));
  RoundSink sink{nullptr, nullptr, o16, static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), lse};
  hipError_t e = d == 64 ? launch_fast64<64, kSinkCompact>(qk, v, perm, bh, n_rounds - 1, 0, s, sink, stream)
                         : launch_fast64<128, kSinkCompact>(qk, v, perm, bh, n_rounds - 1, 0, s, sink, stream);
  if (e == hipSuccess && mark != nullptr) e = hipEventRecord(*mark, stream);
  if (e != hipSuccess) return e;
  switch (n_rounds) {
    case 1: return launch_final<sink_final_prefetch(0)>(qk, v, perm, bh, d, s, sink, stream);
    case 2: return launch_final<sink_final_prefetch(1)>(qk, v, perm, bh, d, s, sink, stream);
    case 4: return launch_final<sink_final_prefetch(3)>(qk, v, perm, bh, d, s, sink, stream);
    case 8:   // seven prefetched rows fit the register budget at d = 64 only
      if (d == 64) return launch_fast64<64, sink_final_prefetch(7)>(qk, v, perm, bh, 1, 7, s, sink, stream);
      return launch_final<kSinkFinal>(qk, v, perm, bh, d, s, sink, stream);
    default: return launch_final<kSinkFinal>(qk, v, perm, bh, d, s, sink, stream);
  }
}

}  // namespace rlsh
